"""The oracle's pins must catch plausible slips: each planted mutant fails one.

Each case plants one mistake in a private copy of ``oracle/eager_oracle.c``
(on the CPU, in a temporary directory), builds it, points the oracle wrapper at
the mutant and runs the pin tests of ``test_oracle_pins.py`` against it.  At
least one pin must fail for every mutant; the unmodified source must pass all.
"""
import ctypes
import inspect
import os
import subprocess

import pytest

import oracle
from oracle import build as obuild
from tests import test_oracle_pins as pins

MUTANTS = {
    "gdn_sign_of_correction": ("u[j] = b * (v[j] - a * y[j]);", "u[j] = b * (v[j] + a * y[j]);"),
    "gdn_alpha_dropped_in_correction": ("u[j] = b * (v[j] - a * y[j]);", "u[j] = b * (v[j] - y[j]);"),
    "gdn_transposed_read": (
        "for (int c = 0; c < dk; ++c) acc += S[(size_t)c * dv + j] * k[c];\n        y[j] = acc;\n    }\n    for (int j = 0; j < dv; ++j) u[j] = b * (v[j] - a",
        "for (int c = 0; c < dk; ++c) acc += S[(size_t)j * dk + c] * k[c];\n        y[j] = acc;\n    }\n    for (int j = 0; j < dv; ++j) u[j] = b * (v[j] - a"),
    "gdn_output_reads_key": (
        "S[(size_t)c * dv + j] = a * S[(size_t)c * dv + j] + k[c] * u[j];\n    for (int j = 0; j < dv; ++j) {\n        double acc = 0.0;\n        for (int c = 0; c < dk; ++c) acc += S[(size_t)c * dv + j] * q[c];",
        "S[(size_t)c * dv + j] = a * S[(size_t)c * dv + j] + k[c] * u[j];\n    for (int j = 0; j < dv; ++j) {\n        double acc = 0.0;\n        for (int c = 0; c < dk; ++c) acc += S[(size_t)c * dv + j] * k[c];"),
    "kda_decay_index_slip": ("S[(size_t)c * dv + j] *= a[c];", "S[(size_t)c * dv + j] *= a[(c + 1) % dk];"),
    "kda_beta_dropped": ("u[j] = b * (v[j] - y[j]);", "u[j] = (v[j] - y[j]); (void)b;"),
    "rwkv6_bonus_dropped": ("s += r[c] * bonus[c] * k[c];", "s += r[c] * k[c]; (void)bonus;"),
    "rwkv6_update_uses_r": ("S[(size_t)c * dv + j] + k[c] * v[j];", "S[(size_t)c * dv + j] + r[c] * v[j];"),
    "rwkv6_decay_on_value_axis": (
        "S[(size_t)c * dv + j] = w[c] * S[(size_t)c * dv + j] + k[c] * v[j];",
        "S[(size_t)c * dv + j] = w[j % dk] * S[(size_t)c * dv + j] + k[c] * v[j];"),
    "rwkv6_output_after_update": (
        "    double s = 0.0;\n    for (int c = 0; c < dk; ++c) s += r[c] * bonus[c] * k[c];\n    for (int j = 0; j < dv; ++j) {\n        double acc = 0.0;\n        for (int c = 0; c < dk; ++c) acc += r[c] * S[(size_t)c * dv + j];\n        o[j] = acc + s * v[j];\n    }\n    for (int c = 0; c < dk; ++c)\n        for (int j = 0; j < dv; ++j)\n            S[(size_t)c * dv + j] = w[c] * S[(size_t)c * dv + j] + k[c] * v[j];",
        "    double s = 0.0;\n    for (int c = 0; c < dk; ++c) s += r[c] * bonus[c] * k[c];\n    for (int c = 0; c < dk; ++c)\n        for (int j = 0; j < dv; ++j)\n            S[(size_t)c * dv + j] = w[c] * S[(size_t)c * dv + j] + k[c] * v[j];\n    for (int j = 0; j < dv; ++j) {\n        double acc = 0.0;\n        for (int c = 0; c < dk; ++c) acc += r[c] * S[(size_t)c * dv + j];\n        o[j] = acc + s * v[j];\n    }"),
    "checkpoint_off_by_one": ("save_checkpoints(jb, n, t + 1, S);", "save_checkpoints(jb, n, t, S);"),
}


def _pin_cases():
    """(name, callable) for every pin, with each parametrisation expanded."""
    cases = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_") or name == "test_rejects_bad_arguments":
            continue
        marks = getattr(fn, "pytestmark", [])
        grids = [m for m in marks if m.name == "parametrize"]
        combos = [{}]
        for m in grids:
            argnames = [a.strip() for a in m.args[0].split(",")] if isinstance(m.args[0], str) else list(m.args[0])
            new = []
            for c in combos:
                for val in m.args[1]:
                    vals = val if len(argnames) > 1 else (val,)
                    d = dict(c)
                    d.update(zip(argnames, vals))
                    new.append(d)
            combos = new
        for c in combos:
            cases.append((f"{name}{c}", fn, c))
    return cases


def _load_lib(path):
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int)
    lib.oracle_eager_run.restype = ctypes.c_int
    lib.oracle_eager_run.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, ip, ctypes.c_int, ctypes.c_int]
    return lib


def _failures_with(src_text, tmp_path, tag):
    c_path = os.path.join(tmp_path, f"{tag}.c")
    so_path = os.path.join(tmp_path, f"lib{tag}.so")
    with open(c_path, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", so_path, c_path],
                   check=True)
    saved = oracle._lib
    oracle._lib = _load_lib(so_path)
    failed = []
    try:
        for name, fn, kw in _pin_cases():
            try:
                fn(**kw)
            except AssertionError:
                failed.append(name)
    finally:
        oracle._lib = saved
    return failed


@pytest.fixture(scope="module")
def source():
    with open(obuild.SRC) as f:
        return f.read()


def test_unmodified_source_passes_every_pin(source, tmp_path):
    assert _failures_with(source, str(tmp_path), "clean") == []


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_mutant_is_caught(mutant, source, tmp_path):
    old, new = MUTANTS[mutant]
    assert source.count(old) == 1, f"mutation site of {mutant} not unique in the oracle source"
    failed = _failures_with(source.replace(old, new), str(tmp_path), mutant)
    assert failed, f"no pin caught the planted slip {mutant}"
