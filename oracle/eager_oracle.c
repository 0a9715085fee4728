/*
 * eager_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, fp64 CPU implementation of the eager dense recurrent-state
 * decode step for three linear-attention operators.  It exists to check the
 * GPU path and is never part of it: only the tests, the smoke check and the
 * CPU-baseline leg of the benchmark may load it.  It shares no code, header,
 * table or constant with the HIP library.
 *
 * What it computes.  DeltaLog never changes the model's recurrence; the
 * logical state it keeps must equal the dense state eager decoding would
 * hold after every token (DeltaLog abstract, as reproduced on the scholarbro
 * "Raven" and "DART" pages; gist.science summary, sections "Metodologia" and
 * "Contributi Chiave").  So the oracle for the whole decode path is the eager
 * recurrence itself, written out element by element with no blocking,
 * fusion or reordering.
 *
 * State layout: one head's state is S[c][j], c = key channel (0..dk-1),
 * j = value channel (0..dv-1), j contiguous -- the [B,H,dk,dv] tensor named
 * in the gist.science summary, section "Problema".  The three operators are
 * named in section "Operatori" of that summary (GDN: scalar per-head decay
 * with the delta-rule correction; KDA: per-key decay with the delta-rule
 * correction; RWKV6: per-key decay with raw value updates).  The pages do
 * not print the formulas; the standard operator definitions are used:
 *
 *   GDN   S_t = a_t S_{t-1} + b_t k_t (v_t - a_t S_{t-1}^T k_t)^T,
 *         o_t = S_t^T q_t                          (a_t scalar in (0,1])
 *   KDA   the same with S_{t-1} replaced by diag(a_t) S_{t-1},
 *         a_t a per-key-channel vector in (0,1]^dk
 *   RWKV6 o_t = S_{t-1}^T r_t + (sum_c r_t[c] u[c] k_t[c]) v_t,
 *         S_t = diag(w_t) S_{t-1} + k_t v_t^T      (u = per-head bonus)
 *
 * There is no scaling of q (o_t = S_t^T q_t exactly) and GDN/KDA output is
 * read from the post-update state, RWKV6 output from the pre-update state
 * plus the bonus term.
 */
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_GDN = 0, ORACLE_KDA = 1, ORACLE_RWKV6 = 2 };

typedef struct {
    int op, N, dk, dv, T;
    const double *q, *k, *v, *beta, *decay, *bonus, *S0;
    double *out, *ufac, *states;
    const int *chk;
    int nchk;
    int head_begin, head_end;
    int status;
} oracle_job;

/* Save S into every checkpoint slot whose step equals t. */
static void save_checkpoints(const oracle_job *jb, int n, int t, const double *S) {
    size_t hs = (size_t)jb->dk * jb->dv;
    for (int m = 0; m < jb->nchk; ++m)
        if (jb->chk[m] == t && jb->states)
            memcpy(jb->states + ((size_t)m * jb->N + n) * hs, S, hs * sizeof(double));
}

/* GDN, one token: y = S^T k; u = b (v - a y); S = a S + k u^T; o = S^T q. */
static void gdn_step(int dk, int dv, double *S, double *y, double *u,
                     const double *q, const double *k, const double *v,
                     double b, double a, double *o) {
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int c = 0; c < dk; ++c) acc += S[(size_t)c * dv + j] * k[c];
        y[j] = acc;
    }
    for (int j = 0; j < dv; ++j) u[j] = b * (v[j] - a * y[j]);
    for (int c = 0; c < dk; ++c)
        for (int j = 0; j < dv; ++j)
            S[(size_t)c * dv + j] = a * S[(size_t)c * dv + j] + k[c] * u[j];
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int c = 0; c < dk; ++c) acc += S[(size_t)c * dv + j] * q[c];
        o[j] = acc;
    }
}

/* KDA, one token: S = diag(a) S; y = S^T k; u = b (v - y); S += k u^T; o = S^T q. */
static void kda_step(int dk, int dv, double *S, double *y, double *u,
                     const double *q, const double *k, const double *v,
                     double b, const double *a, double *o) {
    for (int c = 0; c < dk; ++c)
        for (int j = 0; j < dv; ++j) S[(size_t)c * dv + j] *= a[c];
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int c = 0; c < dk; ++c) acc += S[(size_t)c * dv + j] * k[c];
        y[j] = acc;
    }
    for (int j = 0; j < dv; ++j) u[j] = b * (v[j] - y[j]);
    for (int c = 0; c < dk; ++c)
        for (int j = 0; j < dv; ++j) S[(size_t)c * dv + j] += k[c] * u[j];
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int c = 0; c < dk; ++c) acc += S[(size_t)c * dv + j] * q[c];
        o[j] = acc;
    }
}

/* RWKV6, one token: o = S^T r + (sum_c r u k) v; S = diag(w) S + k v^T. */
static void rwkv6_step(int dk, int dv, double *S,
                       const double *r, const double *k, const double *v,
                       const double *w, const double *bonus, double *o) {
    double s = 0.0;
    for (int c = 0; c < dk; ++c) s += r[c] * bonus[c] * k[c];
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int c = 0; c < dk; ++c) acc += r[c] * S[(size_t)c * dv + j];
        o[j] = acc + s * v[j];
    }
    for (int c = 0; c < dk; ++c)
        for (int j = 0; j < dv; ++j)
            S[(size_t)c * dv + j] = w[c] * S[(size_t)c * dv + j] + k[c] * v[j];
}

/* Run the T-token trajectory of heads [head_begin, head_end). */
static void *run_heads(void *arg) {
    oracle_job *jb = (oracle_job *)arg;
    const int N = jb->N, dk = jb->dk, dv = jb->dv;
    const size_t hs = (size_t)dk * dv;
    double *S = (double *)malloc(hs * sizeof(double));
    double *y = (double *)malloc((size_t)dv * sizeof(double));
    double *u = (double *)malloc((size_t)dv * sizeof(double));
    if (!S || !y || !u) {
        free(S); free(y); free(u);
        jb->status = -1;
        return NULL;
    }
    for (int n = jb->head_begin; n < jb->head_end; ++n) {
        memcpy(S, jb->S0 + (size_t)n * hs, hs * sizeof(double));
        save_checkpoints(jb, n, 0, S);
        for (int t = 0; t < jb->T; ++t) {
            const size_t tn = (size_t)t * N + n;
            const double *q = jb->q + tn * dk;
            const double *k = jb->k + tn * dk;
            const double *v = jb->v + tn * dv;
            double *o = jb->out + tn * dv;
            if (jb->op == ORACLE_GDN) {
                gdn_step(dk, dv, S, y, u, q, k, v, jb->beta[tn], jb->decay[tn], o);
            } else if (jb->op == ORACLE_KDA) {
                kda_step(dk, dv, S, y, u, q, k, v, jb->beta[tn], jb->decay + tn * dk, o);
            } else {
                rwkv6_step(dk, dv, S, q, k, v, jb->decay + tn * dk, jb->bonus + (size_t)n * dk, o);
                memcpy(u, v, (size_t)dv * sizeof(double));
            }
            if (jb->ufac) memcpy(jb->ufac + tn * dv, u, (size_t)dv * sizeof(double));
            save_checkpoints(jb, n, t + 1, S);
        }
    }
    free(S); free(y); free(u);
    jb->status = 0;
    return NULL;
}

/*
 * oracle_eager_run -- run N independent heads for T tokens.
 *
 *   op      0 = GDN, 1 = KDA, 2 = RWKV6
 *   q       [T][N][dk]   q_t (GDN/KDA) or r_t (RWKV6)
 *   k       [T][N][dk]
 *   v       [T][N][dv]
 *   beta    [T][N]       GDN/KDA only (may be NULL for RWKV6)
 *   decay   [T][N] (GDN)  or  [T][N][dk] (KDA, RWKV6)
 *   bonus   [N][dk]      RWKV6 only: the bonus of each head's own attention head
 *   S0      [N][dk][dv]  initial state
 *   out     [T][N][dv]   output o_t of every token
 *   ufac    [T][N][dv]   optional: the value-side factor of every token
 *                        (u_t for GDN/KDA, v_t for RWKV6); NULL to skip
 *   states  [nchk][N][dk][dv]  optional: the state after chk[m] tokens
 *                        (0 <= chk[m] <= T; 0 is S0); NULL to skip
 *   nthreads  worker threads over disjoint head ranges (<= 0 means 1)
 *
 * Returns 0 on success, -1 on bad arguments or allocation failure.
 */
int oracle_eager_run(int op, int N, int dk, int dv, int T,
                     const double *q, const double *k, const double *v,
                     const double *beta, const double *decay, const double *bonus,
                     const double *S0, double *out, double *ufac, double *states,
                     const int *chk, int nchk, int nthreads) {
    if (op < ORACLE_GDN || op > ORACLE_RWKV6 || N < 0 || dk <= 0 || dv <= 0 || T < 0)
        return -1;
    if (!q || !k || !v || !decay || !S0 || !out) return -1;
    if (op != ORACLE_RWKV6 && !beta) return -1;
    if (op == ORACLE_RWKV6 && !bonus) return -1;
    if (nchk > 0 && (!chk || !states)) return -1;
    if (nthreads <= 0) nthreads = 1;
    if (nthreads > N) nthreads = N > 0 ? N : 1;

    oracle_job *jobs = (oracle_job *)calloc((size_t)nthreads, sizeof(oracle_job));
    pthread_t *tids = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tids) {
        free(jobs); free(tids);
        return -1;
    }
    int status = 0;
    for (int w = 0; w < nthreads; ++w) {
        oracle_job *jb = &jobs[w];
        jb->op = op; jb->N = N; jb->dk = dk; jb->dv = dv; jb->T = T;
        jb->q = q; jb->k = k; jb->v = v; jb->beta = beta; jb->decay = decay;
        jb->bonus = bonus; jb->S0 = S0; jb->out = out; jb->ufac = ufac;
        jb->states = states; jb->chk = chk; jb->nchk = nchk;
        jb->head_begin = (int)((long long)N * w / nthreads);
        jb->head_end = (int)((long long)N * (w + 1) / nthreads);
    }
    unsigned char *joined = (unsigned char *)calloc((size_t)nthreads, 1);
    if (!joined) {
        free(jobs); free(tids);
        return -1;
    }
    for (int w = 1; w < nthreads; ++w) {
        if (pthread_create(&tids[w], NULL, run_heads, &jobs[w]) == 0)
            joined[w] = 1;
        else
            run_heads(&jobs[w]); /* no thread available: run this range inline */
    }
    run_heads(&jobs[0]);
    for (int w = 1; w < nthreads; ++w)
        if (joined[w]) pthread_join(tids[w], NULL);
    for (int w = 0; w < nthreads; ++w)
        if (jobs[w].status != 0) status = -1;
    free(joined);
    free(jobs);
    free(tids);
    return status;
}
