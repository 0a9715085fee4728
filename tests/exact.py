"""Exact rational closed forms of the three recurrences (tests only).

These are not the oracle's step-by-step recursion retyped: they expand the
whole trajectory into products of transition matrices (delta rules) or into
decayed sums of outer products (RWKV6), in Python ``Fraction`` arithmetic, so
they pin the fp64 oracle on tiny inputs without sharing its evaluation order.

Orientation: a state is a dk x dv matrix S[c][j] (key channel c, value
channel j); vectors are lists.

  GDN/KDA   M_t = (I - b_t k_t k_t^T) diag(a_t)          (dk x dk)
            S_t = M_t ... M_1 S_0 + sum_s M_t ... M_{s+1} b_s k_s v_s^T
            o_t = S_t^T q_t
  RWKV6     S_t = diag(prod_{s<=t} w_s) S_0
                  + sum_{s<=t} diag(prod_{s<j<=t} w_j) k_s v_s^T
            o_t = S_{t-1}^T r_t + (sum_c r_t[c] u[c] k_t[c]) v_t
"""
from fractions import Fraction


def eye(n):
    return [[Fraction(int(i == j)) for j in range(n)] for i in range(n)]


def matmul(A, B):
    n, m, p = len(A), len(B), len(B[0])
    return [[sum((A[i][l] * B[l][j] for l in range(m)), Fraction(0)) for j in range(p)]
            for i in range(n)]


def matadd(A, B):
    return [[a + b for a, b in zip(ra, rb)] for ra, rb in zip(A, B)]


def outer(x, y):
    return [[a * b for b in y] for a in x]


def scale(s, A):
    return [[s * a for a in row] for row in A]


def transpose_matvec(S, x):
    """S^T x for S of shape dk x dv and x of length dk."""
    dk, dv = len(S), len(S[0])
    return [sum((S[c][j] * x[c] for c in range(dk)), Fraction(0)) for j in range(dv)]


def diag(d):
    n = len(d)
    return [[d[i] if i == j else Fraction(0) for j in range(n)] for i in range(n)]


def delta_transition(k, b, a):
    """M = (I - b k k^T) diag(a)."""
    dk = len(k)
    P = matadd(eye(dk), scale(-b, outer(k, k)))
    return matmul(P, diag(a))


def delta_closed_form(S0, qs, ks, vs, bs, decays):
    """States S_1..S_T and outputs o_1..o_T of GDN/KDA by the unrolled closed form.

    ``decays[t]`` is the per-key-channel vector a_t (GDN passes alpha_t * ones).
    """
    T = len(qs)
    Ms = [delta_transition(ks[t], bs[t], decays[t]) for t in range(T)]
    states, outs = [], []
    dk = len(S0)
    for t in range(T):
        # prefix product M_t ... M_1 and the injected terms
        P = eye(dk)
        for s in range(t + 1):
            P = matmul(Ms[s], P)
        S = matmul(P, S0)
        for s in range(t + 1):
            Q = eye(dk)
            for j in range(s + 1, t + 1):
                Q = matmul(Ms[j], Q)
            S = matadd(S, matmul(Q, scale(bs[s], outer(ks[s], vs[s]))))
        states.append(S)
        outs.append(transpose_matvec(S, qs[t]))
    return states, outs


def rwkv6_closed_form(S0, rs, ks, vs, ws, bonus):
    """States S_1..S_T and outputs o_1..o_T of RWKV6 by the decayed-sum closed form."""
    T = len(rs)
    dk, dv = len(S0), len(S0[0])

    def state_after(t):
        # tokens 0..t-1 have been absorbed (t = 0 is S0)
        prod_all = [Fraction(1)] * dk
        for s in range(t):
            prod_all = [p * w for p, w in zip(prod_all, ws[s])]
        S = matmul(diag(prod_all), S0)
        for s in range(t):
            prod = [Fraction(1)] * dk
            for j in range(s + 1, t):
                prod = [p * w for p, w in zip(prod, ws[j])]
            S = matadd(S, matmul(diag(prod), outer(ks[s], vs[s])))
        return S

    states, outs = [], []
    for t in range(T):
        prev = state_after(t)
        bon = sum((rs[t][c] * bonus[c] * ks[t][c] for c in range(dk)), Fraction(0))
        o = transpose_matvec(prev, rs[t])
        outs.append([o[j] + bon * vs[t][j] for j in range(dv)])
        states.append(state_after(t + 1))
    return states, outs
