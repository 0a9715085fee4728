"""fp64 CPU oracle for the recurrent-state decode step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import this package.  The GPU library never calls it
and shares no code with it.

The oracle is the eager dense recurrence (see ``eager_oracle.c`` for the
formulas and the passages they follow).  DeltaLog's claim is that its
base-plus-log state is, after every token, the same dense state eager decoding
holds (DeltaLog abstract on the scholarbro "Raven"/"DART" pages; gist.science
summary, "Contributi Chiave"), so this single function is the reference for
outputs, compact factors and materialised states alike.

Parity status of each function: pinned by ``tests/test_oracle_pins.py``
(exact rational closed forms on tiny inputs, special cases that reduce to
textbook formulas, invariants).  No function here is "parity unpinned".
"""
import ctypes
import os

import numpy as np

from . import build as _build

OPS = {"gdn": 0, "kda": 1, "rwkv6": 2}

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int)
        lib.oracle_eager_run.restype = ctypes.c_int
        lib.oracle_eager_run.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, ip, ctypes.c_int, ctypes.c_int]
        _lib = lib
    return _lib


def _f64(x, shape):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    if a.shape != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {a.shape}")
    return a


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def eager_run(op, q, k, v, beta, decay, bonus, S0, chk_steps=(), want_factors=False,
              nthreads=1):
    """Run the eager fp64 recurrence over N independent heads.

    Shapes (numpy-convertible, upcast exactly to float64):
      q, k: [T, N, dk]   (q is r for RWKV6)
      v:    [T, N, dv]
      beta: [T, N] for GDN/KDA, None for RWKV6
      decay: [T, N] for GDN (alpha), [T, N, dk] for KDA (a) and RWKV6 (w)
      bonus: [N, dk] for RWKV6 (each head's own bonus row), None otherwise
      S0:   [N, dk, dv]
      chk_steps: token counts t (0..T) after which the state is returned

    Returns a dict with ``out`` [T, N, dv], ``states`` [len(chk_steps), N, dk, dv]
    and, if ``want_factors``, ``factors`` [T, N, dv] (u_t for GDN/KDA, v_t for
    RWKV6).
    """
    if op not in OPS:
        raise ValueError(f"unknown op {op!r}")
    code = OPS[op]
    q = np.asarray(q)
    T, N, dk = q.shape
    dv = np.asarray(v).shape[2]
    q = _f64(q, (T, N, dk))
    k = _f64(k, (T, N, dk))
    v = _f64(v, (T, N, dv))
    if op == "gdn":
        decay = _f64(decay, (T, N))
    else:
        decay = _f64(decay, (T, N, dk))
    beta = None if op == "rwkv6" else _f64(beta, (T, N))
    bonus = _f64(bonus, (N, dk)) if op == "rwkv6" else None
    S0 = _f64(S0, (N, dk, dv))
    chk = np.ascontiguousarray(np.asarray(list(chk_steps), dtype=np.int32))
    if chk.size and (chk.min() < 0 or chk.max() > T):
        raise ValueError("checkpoint steps must lie in [0, T]")
    out = np.zeros((T, N, dv), dtype=np.float64)
    fac = np.zeros((T, N, dv), dtype=np.float64) if want_factors else None
    states = np.zeros((chk.size, N, dk, dv), dtype=np.float64) if chk.size else None
    lib = _load()
    rc = lib.oracle_eager_run(
        code, N, dk, dv, T, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(decay),
        _ptr(bonus), _ptr(S0), _ptr(out), _ptr(fac), _ptr(states),
        chk.ctypes.data_as(ctypes.POINTER(ctypes.c_int)) if chk.size else None,
        int(chk.size), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_eager_run failed with status {rc}")
    res = {"out": out, "states": states if states is not None else
           np.zeros((0, N, dk, dv))}
    if want_factors:
        res["factors"] = fac
    return res
