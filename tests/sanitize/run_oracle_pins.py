"""Run every pin of the oracle against another build of its library.

Usage: python run_oracle_pins.py LIB.so -- used by test_sanitizers.py to run
the pins against the oracle compiled with the address and undefined-
behaviour sanitizers, in a process of its own (the sanitizer runtime must be
loaded first).  Prints the number of pins run and exits 1 if any failed.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from tests import test_oracle_mutants as mutants  # noqa: E402


def main():
    oracle._lib = mutants._load_lib(sys.argv[1])
    failed, cases = [], mutants._pin_cases()
    for name, fn, kw in cases:
        try:
            fn(**kw)
        except AssertionError as e:
            failed.append(f"{name}: {e}")
    print(f"oracle pins under sanitizers: {len(cases) - len(failed)} of {len(cases)} passed", flush=True)
    for f in failed:
        print("FAILED", f, flush=True)
    sys.exit(1 if failed else 0)


if __name__ == "__main__":
    main()
