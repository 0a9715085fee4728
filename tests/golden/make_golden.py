"""Write ``tests/golden/oracle_dyadic.json`` by calling only ``oracle/``.

The DeltaLog pages print no worked numeric example (the summary page says its
equations were never rendered, and every results figure survives only as a
caption), so there is no printed value to store.  This fixture is a regression
anchor instead: tiny dyadic-rational inputs (exact in binary), the oracle's
fp64 outputs and final states as hex floats.  The test that reads it also
checks the stored values against the exact rational closed forms.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import random
import sys
from fractions import Fraction

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402

OUT = os.path.join(HERE, "oracle_dyadic.json")


def dyadic_case(op, dk, dv, T, seed):
    """Inputs as fraction strings; every value is m / 2^p, so exact in fp64."""
    rng = random.Random(seed)

    def vec(n, lo, hi, den):
        return [str(Fraction(rng.randint(lo, hi), den)) for _ in range(n)]

    case = {"op": op, "dk": dk, "dv": dv, "T": T,
            "S0": [vec(dv, -8, 8, 16) for _ in range(dk)],
            "q": [vec(dk, -8, 8, 8) for _ in range(T)],
            "k": [vec(dk, -4, 4, 8) for _ in range(T)],
            "v": [vec(dv, -8, 8, 8) for _ in range(T)]}
    if op == "rwkv6":
        case["decay"] = [vec(dk, 9, 16, 16) for _ in range(T)]
        case["bonus"] = vec(dk, -8, 8, 16)
    else:
        case["beta"] = [str(Fraction(rng.randint(1, 16), 16)) for _ in range(T)]
        if op == "gdn":
            case["decay"] = [str(Fraction(rng.randint(9, 16), 16)) for _ in range(T)]
        else:
            case["decay"] = [vec(dk, 9, 16, 16) for _ in range(T)]
    return case


def as_f64(x):
    if isinstance(x, list):
        return np.array([as_f64(e) for e in x], dtype=np.float64)
    return float(Fraction(x))


def run_case(case):
    op, T = case["op"], case["T"]
    q = as_f64(case["q"])[:, None, :]
    k = as_f64(case["k"])[:, None, :]
    v = as_f64(case["v"])[:, None, :]
    if op == "gdn":
        decay = as_f64(case["decay"])[:, None]
    else:
        decay = as_f64(case["decay"])[:, None, :]
    beta = None if op == "rwkv6" else as_f64(case["beta"])[:, None]
    bonus = as_f64(case["bonus"])[None, :] if op == "rwkv6" else None
    S0 = as_f64(case["S0"])[None]
    return oracle.eager_run(op, q, k, v, beta, decay, bonus, S0, chk_steps=[T])


def main():
    cases = [dyadic_case("gdn", 3, 2, 4, 7), dyadic_case("kda", 2, 3, 4, 8),
             dyadic_case("rwkv6", 3, 4, 4, 9)]
    for case in cases:
        res = run_case(case)
        case["out_hex"] = [[float(x).hex() for x in row] for row in res["out"][:, 0]]
        case["final_state_hex"] = [[float(x).hex() for x in row] for row in res["states"][0, 0]]
    doc = {"source": "written by tests/golden/make_golden.py from oracle/ only",
           "note": "the DeltaLog pages print no worked numeric example; regression anchor",
           "cases": cases}
    with open(OUT, "w") as f:
        json.dump(doc, f, indent=1)
    print(OUT)


if __name__ == "__main__":
    main()
