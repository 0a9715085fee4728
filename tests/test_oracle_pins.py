"""Pins of the fp64 CPU oracle against mathematics it does not share code with.

Every test here runs on the CPU.  Each one is chosen so that a plausible slip
in ``oracle/eager_oracle.c`` -- a dropped term, a wrong sign, a transposed
operand (dk != dv everywhere below), the pre- vs post-update state in an
output, a decay applied to the wrong axis -- fails at least one of them:

* exact rational closed forms on tiny inputs (``tests/exact.py``);
* special cases that reduce to textbook results: pure decay (beta = 0), the
  delta rule's exact overwrite / retrieval, KDA with a scalar decay equal to
  GDN, RWKV6 without decay equal to causal linear attention plus a diagonal
  bonus (a handful of numpy matrix products);
* invariants: linearity of the delta rules in (S0, v), the value factor
  reproducing the state increment, head independence and thread invariance.
"""
import random
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import exact


def _frac_vec(rng, n, lo=-8, hi=8, den=8):
    return [Fraction(rng.randint(lo, hi), den) for _ in range(n)]


def _decay_vec(rng, n):
    # dyadic values in (0, 1]: exactly representable in fp64
    return [Fraction(rng.randint(9, 16), 16) for _ in range(n)]


def _to_np(x):
    return np.array([[float(a) for a in row] for row in x]) if isinstance(x[0], list) \
        else np.array([float(a) for a in x])


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
@pytest.mark.parametrize("dk,dv,T,seed", [(3, 2, 5, 1), (2, 4, 6, 2), (4, 3, 4, 3)])
def test_exact_closed_form(op, dk, dv, T, seed):
    """fp64 oracle == exact rational closed form (<= 1e-12 relative) on tiny inputs."""
    rng = random.Random(1000 * seed + dk * 10 + dv)
    S0 = [_frac_vec(rng, dv, den=16) for _ in range(dk)]
    qs = [_frac_vec(rng, dk) for _ in range(T)]
    ks = [_frac_vec(rng, dk, lo=-4, hi=4) for _ in range(T)]
    vs = [_frac_vec(rng, dv) for _ in range(T)]
    if op == "rwkv6":
        ws = [_decay_vec(rng, dk) for _ in range(T)]
        bonus = _frac_vec(rng, dk, den=16)
        states, outs = exact.rwkv6_closed_form(S0, qs, ks, vs, ws, bonus)
        decay = np.array([[_to_np(w)] for w in ws])
        beta = None
        bon = _to_np(bonus)[None, :]
    else:
        bs = [Fraction(rng.randint(1, 16), 16) for _ in range(T)]
        if op == "gdn":
            al = [Fraction(rng.randint(9, 16), 16) for _ in range(T)]
            decs = [[a] * dk for a in al]
            decay = np.array([[float(a)] for a in al])
        else:
            decs = [_decay_vec(rng, dk) for _ in range(T)]
            decay = np.array([[_to_np(a)] for a in decs])
        states, outs = exact.delta_closed_form(S0, qs, ks, vs, bs, decs)
        beta = np.array([[float(b)] for b in bs])
        bon = None
    q = np.array([[_to_np(x)] for x in qs])
    k = np.array([[_to_np(x)] for x in ks])
    v = np.array([[_to_np(x)] for x in vs])
    res = oracle.eager_run(op, q, k, v, beta, decay, bon, _to_np(S0)[None],
                           chk_steps=list(range(1, T + 1)))
    for t in range(T):
        assert _rel(res["out"][t, 0], _to_np(outs[t])) <= 1e-12, f"output t={t}"
        assert _rel(res["states"][t, 0], _to_np(states[t])) <= 1e-12, f"state t={t}"


def _rand_inputs(op, T, N, dk, dv, seed, unit_keys=True):
    g = np.random.default_rng(seed)
    q = g.standard_normal((T, N, dk))
    k = g.standard_normal((T, N, dk))
    if unit_keys:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = g.standard_normal((T, N, dv))
    beta = 1.0 / (1.0 + np.exp(-g.standard_normal((T, N))))
    if op == "gdn":
        decay = g.uniform(0.9, 1.0, (T, N))
    else:
        decay = g.uniform(0.5, 1.0, (T, N, dk))
    bonus = 0.1 * g.standard_normal((N, dk))
    S0 = 0.02 * g.standard_normal((N, dk, dv))
    return q, k, v, beta, decay, bonus, S0


def test_gdn_pure_decay():
    """beta = 0: S_t = (prod alpha) S0 and o_t = (prod_{s<=t} alpha_s) S0^T q_t."""
    T, N, dk, dv = 7, 3, 5, 6
    q, k, v, beta, decay, _, S0 = _rand_inputs("gdn", T, N, dk, dv, 11)
    beta[:] = 0.0
    res = oracle.eager_run("gdn", q, k, v, beta, decay, None, S0, chk_steps=[T])
    cum = np.cumprod(decay, axis=0)  # [T, N]
    for t in range(T):
        want = cum[t][:, None] * np.einsum("ncj,nc->nj", S0, q[t])
        assert _rel(res["out"][t], want) <= 1e-13
    assert _rel(res["states"][0], cum[-1][:, None, None] * S0) <= 1e-13


@pytest.mark.parametrize("op", ["gdn", "kda"])
def test_delta_rule_exact_retrieval(op):
    """decay = 1, beta = 1, |k| = 1: the just-written value is read back, S_t^T k_t = v_t."""
    T, N, dk, dv = 9, 2, 8, 5
    q, k, v, beta, decay, _, S0 = _rand_inputs(op, T, N, dk, dv, 12)
    beta[:] = 1.0
    decay[:] = 1.0
    res = oracle.eager_run(op, q, k, v, beta, decay, None, S0, chk_steps=list(range(1, T + 1)))
    for t in range(T):
        got = np.einsum("ncj,nc->nj", res["states"][t], k[t])
        assert np.max(np.abs(got - v[t])) <= 1e-12


def test_gdn_basis_key_overwrite():
    """beta = 1, k_t = e_c: row c of S_t becomes v_t, every other row is scaled by alpha_t."""
    T, N, dk, dv = 6, 1, 4, 3
    q, k, v, beta, decay, _, S0 = _rand_inputs("gdn", T, N, dk, dv, 13)
    beta[:] = 1.0
    k[:] = 0.0
    rows = [t % dk for t in range(T)]
    for t, c in enumerate(rows):
        k[t, 0, c] = 1.0
    res = oracle.eager_run("gdn", q, k, v, beta, decay, None, S0, chk_steps=list(range(T + 1)))
    for t, c in enumerate(rows):
        prev, cur = res["states"][t, 0], res["states"][t + 1, 0]
        want = decay[t, 0] * prev
        want[c] = v[t, 0]
        assert np.max(np.abs(cur - want)) <= 1e-15


def test_kda_scalar_decay_equals_gdn():
    """KDA with a_t = alpha_t * ones is GDN (fp64 rounding order differs, <= 1e-13)."""
    T, N, dk, dv = 12, 3, 6, 4
    q, k, v, beta, decay, _, S0 = _rand_inputs("gdn", T, N, dk, dv, 14)
    kda_decay = np.repeat(decay[:, :, None], dk, axis=2)
    g = oracle.eager_run("gdn", q, k, v, beta, decay, None, S0, chk_steps=[T])
    kd = oracle.eager_run("kda", q, k, v, beta, kda_decay, None, S0, chk_steps=[T])
    assert _rel(kd["out"], g["out"]) <= 1e-13
    assert _rel(kd["states"], g["states"]) <= 1e-13


def test_rwkv6_no_decay_is_causal_linear_attention():
    """w = 1: O = R S0 + (strict_tril(R K^T) + diag(R diag(u) K^T)) V and S_T = S0 + K^T V."""
    T, N, dk, dv = 10, 2, 5, 7
    r, k, v, _, decay, bonus, S0 = _rand_inputs("rwkv6", T, N, dk, dv, 15, unit_keys=False)
    decay[:] = 1.0
    res = oracle.eager_run("rwkv6", r, k, v, None, decay, bonus, S0, chk_steps=[T])
    for n in range(N):
        R, K, V = r[:, n], k[:, n], v[:, n]
        A = np.tril(R @ K.T, -1) + np.diag(np.diag(R @ np.diag(bonus[n]) @ K.T))
        want = R @ S0[n] + A @ V
        assert _rel(res["out"][:, n], want) <= 1e-13
        assert _rel(res["states"][0, n], S0[n] + K.T @ V) <= 1e-13


def test_rwkv6_decay_acts_on_key_rows():
    """A single RWKV6 step from S0 with k = 0: S_1 = diag(w) S0 (rows, not columns)."""
    T, N, dk, dv = 1, 1, 3, 5
    r, k, v, _, decay, bonus, S0 = _rand_inputs("rwkv6", T, N, dk, dv, 16, unit_keys=False)
    k[:] = 0.0
    res = oracle.eager_run("rwkv6", r, k, v, None, decay, bonus, S0, chk_steps=[1])
    assert _rel(res["states"][0, 0], decay[0, 0][:, None] * S0[0]) <= 1e-15
    assert _rel(res["out"][0, 0], S0[0].T @ r[0, 0]) <= 1e-14


@pytest.mark.parametrize("op", ["gdn", "kda"])
def test_delta_rule_linear_in_state_and_values(op):
    """For fixed keys, queries, beta and decay, the outputs and states are linear in (S0, v)."""
    T, N, dk, dv = 8, 2, 5, 3
    q, k, v, beta, decay, _, S0 = _rand_inputs(op, T, N, dk, dv, 17)
    g = np.random.default_rng(99)
    v2 = g.standard_normal(v.shape)
    S02 = 0.02 * g.standard_normal(S0.shape)
    a = oracle.eager_run(op, q, k, v, beta, decay, None, S0, chk_steps=[T])
    b = oracle.eager_run(op, q, k, v2, beta, decay, None, S02, chk_steps=[T])
    ab = oracle.eager_run(op, q, k, v + v2, beta, decay, None, S0 + S02, chk_steps=[T])
    assert _rel(ab["out"], a["out"] + b["out"]) <= 1e-12
    assert _rel(ab["states"], a["states"] + b["states"]) <= 1e-12


@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_value_factor_is_state_increment(op):
    """S_t - decay(S_{t-1}) = k_t f_t^T, with f_t the returned value factor (u_t or v_t)."""
    T, N, dk, dv = 5, 2, 4, 6
    q, k, v, beta, decay, bonus, S0 = _rand_inputs(op, T, N, dk, dv, 18, unit_keys=op != "rwkv6")
    res = oracle.eager_run(op, q, k, v, None if op == "rwkv6" else beta, decay,
                           bonus if op == "rwkv6" else None, S0,
                           chk_steps=list(range(T + 1)), want_factors=True)
    for t in range(T):
        prev, cur = res["states"][t], res["states"][t + 1]
        if op == "gdn":
            decayed = decay[t][:, None, None] * prev
        else:
            decayed = decay[t][:, :, None] * prev
        inc = np.einsum("nc,nj->ncj", k[t], res["factors"][t])
        assert np.max(np.abs(cur - decayed - inc)) <= 1e-14
    if op == "rwkv6":
        assert np.array_equal(res["factors"], v)


@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_heads_independent_and_thread_invariant(op):
    """A head's trajectory does not depend on the other heads or on the thread split (bitwise)."""
    T, N, dk, dv = 6, 9, 4, 4
    q, k, v, beta, decay, bonus, S0 = _rand_inputs(op, T, N, dk, dv, 19)
    kw = dict(chk_steps=[T])
    be = None if op == "rwkv6" else beta
    bo = bonus if op == "rwkv6" else None
    full1 = oracle.eager_run(op, q, k, v, be, decay, bo, S0, nthreads=1, **kw)
    full4 = oracle.eager_run(op, q, k, v, be, decay, bo, S0, nthreads=4, **kw)
    assert np.array_equal(full1["out"], full4["out"])
    assert np.array_equal(full1["states"], full4["states"])
    sel = [7, 2, 5]
    sub = oracle.eager_run(op, q[:, sel], k[:, sel], v[:, sel],
                           None if be is None else be[:, sel], decay[:, sel],
                           None if bo is None else bo[sel], S0[sel], **kw)
    assert np.array_equal(sub["out"], full1["out"][:, sel])
    assert np.array_equal(sub["states"], full1["states"][:, sel])


def test_rejects_bad_arguments():
    q = np.zeros((2, 1, 3))
    with pytest.raises(ValueError):
        oracle.eager_run("nope", q, q, q, np.zeros((2, 1)), np.zeros((2, 1)), None, np.zeros((1, 3, 3)))
    with pytest.raises(ValueError):
        oracle.eager_run("gdn", q, q, q, np.zeros((2, 1)), np.zeros((2, 1)), None,
                         np.zeros((1, 3, 3)), chk_steps=[3])
