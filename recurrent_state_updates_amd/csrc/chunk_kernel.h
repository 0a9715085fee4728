// chunk_kernel.h -- decode K consecutive tokens of every head in one launch.
//
// The single-token step reads the whole base once per token.  When several
// tokens of the same heads are available at once (a draft chain to verify,
// a short prompt continuation), they can share that read: with the base held
// in registers the workgroup forms every token's base products, replays the
// log for each, and resolves the dependence of token t on the earlier tokens
// of the chunk by a forward substitution over the value factors, column by
// column.  The tokens are then appended to the log, or, when the chunk fills
// it, the log's first C entries are folded into the base with one read and
// one write and the tokens past the fold start the new log.  All the tokens'
// products are taken from the base as read (the fold is exact algebra, so a
// token after it sees the same state either way).  A call of more tokens than
// C folds more than once; there (SEG) the fold leaves the new base in the
// registers and the rest of the tokens run as a further segment on an empty
// log.
//
// Algebra (per head; g_t = g_L + sum_{m<=t} log2 decay_m, g_{-1} = g_L; the
// reference point rho_t = g_t for the delta rules, g_{t-1} for RWKV6):
//   base products  Y0_t = Sbar^T (2^{rho_t} k_t) + sum_{i<L} x_i <k_i 2^{rho_t-g_i}, k_t>
//                  Z0_t = the same with q_t (or r_t)
//   delta rules    u_t = beta_t (v_t - Y0_t - sum_{m<t} u_m <k_m 2^{g_t-g_m}, k_t>)
//                  o_t = Z0_t + sum_{m<t} u_m <k_m 2^{g_t-g_m}, q_t> + <k_t, q_t> u_t
//   RWKV6          o_t = Z0_t + sum_{m<t} v_m <k_m 2^{g_{t-1}-g_m}, r_t> + (sum_c r u k) v_t
//   entries        (k_t, u_t or v_t, g_t); when the log fills at token f = C-1-L a fold writes
//                  S = diag(2^{g_f}) Sbar + sum_{e<C} (k_e 2^{g_f-g_e}) x_e^T,
//                  and the tokens t > f become entries t-f-1 of the new log with
//                  their log-decays summed from the fold: g'_t = sum_{f<m<=t} log2 decay_m.
#pragma once

#include "step_kernel.h"

namespace dlk {

// The input-dtype bits of a value that was read from that dtype (exact).
__device__ __forceinline__ void store_raw(float *dst, float x) { *dst = x; }
__device__ __forceinline__ void store_raw(bf16_bits *dst, float x) {
    *dst = static_cast<bf16_bits>(__float_as_uint(x) >> 16);
}

// The same for four consecutive values: the inverse of In4<TIn>::unpack.
template <typename TIn>
struct Pack4;
template <>
struct Pack4<float> {
    __device__ static f4 pack(f4 x) { return x; }
};
template <>
struct Pack4<bf16_bits> {
    __device__ static u2 pack(f4 x) {
        return u2{(__float_as_uint(x.x) >> 16) | (__float_as_uint(x.y) & 0xffff0000u),
                  (__float_as_uint(x.z) >> 16) | (__float_as_uint(x.w) & 0xffff0000u)};
    }
};

// Token pointers of the kernel arguments as opaque scalar values.  The lanes
// of one wave belong to GPW consecutive key-side groups (tokens tb + t0 ..
// tb + t0 + GPW - 1, tb and t0 uniform), so each lane chooses among GPW
// pointers, each a scalar load at a uniform index.  Left visible, the choice would be folded
// back into an index into the argument array, read with a vector load that
// the data load must wait for; the empty asm prevents that.  The result is
// returned as a global-memory pointer (the asm hides where it came from).
template <typename T>
__device__ __forceinline__ T opaque_scalar(T x) {
    asm volatile("" : "+s"(x));
    return x;
}

template <typename T>
using global_ptr = const T __attribute__((address_space(1))) *;

template <typename E, int GPW, typename T>
__device__ __forceinline__ global_ptr<E> group_pick(const T (&arr)[KMAX_TOKENS], int tb, int t0, int K, int g) {
    T r = opaque_scalar(arr[tb + min(t0, K - 1)]);
#pragma unroll
    for (int i = 1; i < GPW; ++i) {
        const T c = opaque_scalar(arr[tb + min(t0 + i, K - 1)]);
        r = g == i ? c : r;
    }
    return (global_ptr<E>)static_cast<const E *>(r);
}

// MM selects the matrix-core form of the token products (phase C) and of the
// fold, at DK = DV = 128 or 64.  A workgroup holds a whole head: waves 2h and
// 2h + 1 hold the 64 columns of column half h (one half at DV = 64), rows
// 0 .. DK/2 - 1 and DK/2 .. DK - 1, 16 lanes per (row, half), so that each
// 16x16x4 k-step is four rows of one half and two waves' products add up per
// column.  The vector form (the other shapes, and calls of fewer than five
// tokens at 64 x 64; see ChunkShape) holds whole heads as row passes.
// Without SEG the call folds at most once (K <= C), at each workgroup's own
// token on a per-slot handle.  SEG runs calls of more tokens than C (C < 8)
// as segments in one workgroup: each fold updates the register tile in place
// and the next tokens start an empty log from it.  The segmented 128 x 128
// matrix-core form asks for three waves per SIMD, which the compiler meets
// without spilling (left alone, KDA settles one register above that, at two
// waves).
template <int OP, typename TIn, int DK, int DV, int TV, int NT, int CMAX, bool MM, bool SEG>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(SEG && MM && DK == 128 && CMAX == 8 ? 3 : 1)))
void chunk_kernel(const ChunkParams p) {
    using G = Geom<DK, DV, TV, NT>;
    constexpr int NTILE = G::NTILE, LPR = G::LPR, RPP = G::RPP, R = G::R, NW = G::NW;
    constexpr int KL = G::KL, EPP = G::EPP;
    constexpr bool GDN = OP == OP_GDN;
    constexpr bool DELTA = OP != OP_RWKV6;
    constexpr int KM = KMAX_TOKENS;
    // entry slots: the old entries and the chunk's tokens (L + K <= C - 1 + KM
    // without SEG; a segment never passes C)
    constexpr int CP = SEG ? CMAX : CMAX + KM;
    constexpr int KPASS_OLD = (CMAX + EPP - 1) / EPP;  // key-side passes over the old entries (L < C)
    constexpr int KPASS = (CP + EPP - 1) / EPP;         // ... over every entry slot
    static_assert(!MM || (DK == DV && (DK == 64 || DK == 128) && TV == DV && NT == 2 * DK && 2 * KM == 16),
                  "matrix-core form: whole square heads of 64 or 128, 2 DK threads, 16 product vectors");
    // s[i] holds tile row rbase + RSTEP * i; xrow[j] holds log entry ebase + ESTEP * j
    constexpr int RSTEP = MM ? 4 : RPP;
    constexpr int ESTEP = MM ? 8 : RPP;
    constexpr int NWR = MM ? 2 : NW;  // row blocks whose products add up in each column
    constexpr int XR = (CMAX + ESTEP - 1) / ESTEP;
    constexpr int GW = GDN ? 1 : DK;  // log-decay values per entry
    using TX = typename std::conditional<DELTA, float, TIn>::type;
    using Raw = typename In4<TIn>::raw;
    using RawX = typename In4<TX>::raw;
    static_assert(KM <= EPP, "one key-side group per token");
    static_assert(64 % KL == 0, "key-side groups do not straddle waves");
    static_assert(R % 4 == 0, "a thread's rows of the scaled vectors are read as float4");
    static_assert(CMAX % 4 == 0 && CP % 4 == 0, "entry slots come in groups of four");
    static_assert(!SEG || CMAX == 8, "segmented calls have C < KMAX_TOKENS");

    // LDS.  Phase B's token-side arrays (keys, queries, log-decays, the scaled
    // vectors) are dead once phase C has read its operands, so in the
    // matrix-core form the per-wave products of phase C reuse their space (a
    // barrier separates the last read from the first write); the vector form
    // reads the scaled vectors while it writes products and keeps both.
    // RWKV6 has no key-side products: no scaled keys, and one side of products
    constexpr int NS = DELTA ? 2 : 1;          // sides of products: keys (delta rules), queries
    constexpr int ZS = NS - 1;                 // index of the query side
    constexpr int SZ_K = KM * DK;              // floats; every size a multiple of 4
    constexpr int SZ_MV0 = DELTA ? SZ_K : 0;
    constexpr int SZ_LG = (KM * GW + 3) & ~3;
    constexpr int SZ_G = ((KM + 1) * GW + 3) & ~3;
    constexpr int SZ_B = 3 * SZ_K + SZ_MV0 + SZ_LG + SZ_G;
    constexpr int SZ_RED = KM * NWR * NS * TV;
    constexpr int POOL = MM ? (SZ_B > SZ_RED ? SZ_B : SZ_RED) : SZ_B + SZ_RED;
    __shared__ __attribute__((aligned(16))) float s_pool[POOL];
    auto &s_k = *reinterpret_cast<float (*)[KM][DK]>(s_pool);                   // token keys
    auto &s_q = *reinterpret_cast<float (*)[KM][DK]>(s_pool + SZ_K);            // token queries (receptances)
    // 2^{rho_t} k_t and 2^{rho_t} q_t (r_t), row r stored at mv_at(r) so that the R
    // rows of one thread (rbase, rbase + RSTEP, ...) are contiguous
    // (s_mv0 is empty for RWKV6 and never read or written there)
    auto &s_mv1 = *reinterpret_cast<float (*)[KM][DK]>(s_pool + 2 * SZ_K);
    auto &s_mv0 = *reinterpret_cast<float (*)[KM][DK]>(s_pool + 3 * SZ_K);
    auto &s_lg = *reinterpret_cast<float (*)[KM][GW]>(s_pool + 3 * SZ_K + SZ_MV0);  // log2 of each token's decay
    auto &s_g = *reinterpret_cast<float (*)[KM + 1][GW]>(s_pool + 3 * SZ_K + SZ_MV0 + SZ_LG);  // g_{t-1} at index t (g_{-1} = g_L)
    auto &s_red = *reinterpret_cast<float (*)[KM][NWR][NS][TV]>(s_pool + (MM ? 0 : SZ_B));
    __shared__ __attribute__((aligned(16))) float s_scale[DK];     // fold: 2^{g_f} per row
    __shared__ __attribute__((aligned(16))) float s_kt[CMAX * DK]; // fold: decayed keys [entry][row], entries < C
    // value factors [entry][col] for the fold (entries < C).  In the
    // matrix-core form row vrow(t) first holds token t's value: L + t up to
    // the fold (phase D reads v_t there and writes u_t in its place), rows
    // from CMAX on for the tokens past it (whose u_t goes to the new log), and
    // row CP for token slots past the chunk; rows C .. CMAX-1 stay free for
    // the fold's zero padding.
    __shared__ __attribute__((aligned(16))) float s_x[(MM ? CP + 1 : CMAX) * TV];
    __shared__ float s_coef[NS][KM][CP];  // per side (keys, queries), token and entry
    __shared__ float s_dot[KM];   // <k_t, q_t> or sum r u k
    __shared__ float s_beta[KM + 1];  // slot KM takes the writes of lanes that hold no token

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    int n, tile;
    block_to_tile<false>(blockIdx.x, p.N, NTILE, n, tile);  // dispatch order (see block_to_tile)
    const int C = p.C;
    // The segment in hand: tokens tb .. tb + K - 1 of the arguments, on a log
    // of L entries, folding it when it fills.
    int tb = 0, L = p.L;
    if (p.slot_base != nullptr) {
        // Per-slot logs: slot b holds its own number of entries and fills at
        // its own token.  The whole workgroup leaves together, before any
        // barrier, when the slot is inactive.
        const int b = n / p.H;
        if (!p.slot_active[b]) return;
        L = (int)((p.step - (unsigned)p.slot_base[b]) % (unsigned)C);
    }
    // with SEG the first segment runs up to the fold (or the call's end)
    int K = SEG ? min(p.K, C - L) : p.K;
    bool fold = L + K >= C;
    int NE = L + K;                     // entries after the segment
    int tf = fold ? C - 1 - L : K - 1;  // the token at which the log fills
    const int last = L > 0 ? L - 1 : 0;
    // the thread's rows of the tile, its four columns (from cq, within the
    // tile) and its rows of the old log's value factors
    const int rbase = MM ? (DK / 2) * (wave & 1) + (lane >> 4) : tid / LPR;
    const int cq = MM ? 64 * (wave >> 1) + 4 * (lane & 15) : 4 * (tid % LPR);
    const int ebase = MM ? 4 * (wave & 1) + (lane >> 4) : tid / LPR;
    const int rblk = MM ? (wave & 1) : wave;
    auto mv_at = [](int row) { return (row % RSTEP) * (DK / RSTEP) + row / RSTEP; };
    const int col0 = tile * TV;
    const int c4 = 4 * (tid % KL);
    const int ke = tid / KL;            // key-side group: token ke, then entries ps*EPP + ke

    // ---------------- Phase A: loads (token ke's key side, the old log, the tile) ----------------
    // group ke takes token min(ke, K-1): groups beyond the chunk load a valid token and ignore it.
    // Every load of the tokens is issued unconditionally and ahead of the tile,
    // so that none of them waits for another (loads complete in issue order).
    constexpr int GPW = 64 / KL;  // key-side groups per wave
    const int t0 = __builtin_amdgcn_readfirstlane(tid >> 6) * GPW;
    const int g = lane / KL;      // ke = t0 + g
    Raw kraw, qraw;
    f4 dec4 = {1.f, 1.f, 1.f, 1.f};
    float alpha = 1.f, beta_t = 0.f;
    TIn vraw[KM];
    // the segment's tokens: group ke's key side, and every token's value at
    // this thread's column (slots past the segment re-read its first token,
    // a valid address, and are never used)
    auto load_tokens = [&]() {
        kraw = *reinterpret_cast<global_ptr<Raw>>(group_pick<TIn, GPW>(p.k, tb, t0, K, g) + (size_t)n * DK + c4);
        qraw = *reinterpret_cast<global_ptr<Raw>>(group_pick<TIn, GPW>(p.q, tb, t0, K, g) + (size_t)n * DK + c4);
        const global_ptr<float> dec_t = group_pick<float, GPW>(p.decay, tb, t0, K, g);
        if (GDN)
            alpha = dec_t[n];
        else
            dec4 = *reinterpret_cast<global_ptr<f4>>(dec_t + (size_t)n * DK + c4);
        if (DELTA) beta_t = group_pick<float, GPW>(p.beta, tb, t0, K, g)[n];
        const void *v0 = opaque_scalar(p.v[tb]);
#pragma unroll
        for (int t = 0; t < KM; ++t) {
            const void *vt = t == 0 ? v0 : opaque_scalar(p.v[min(tb + t, KM - 1)]);
            vt = t < K ? vt : v0;
            vraw[t] = ((global_ptr<TIn>)static_cast<const TIn *>(vt))[(size_t)n * DV + col0 + tid % TV];
        }
    };
    load_tokens();
    f4 bon4 = {0.f, 0.f, 0.f, 0.f};
    if (!DELTA) bon4 = *reinterpret_cast<const f4 *>(p.bonus + (size_t)(n % p.H) * DK + c4);
    float glast_s = 0.f;
    f4 glast4 = {0.f, 0.f, 0.f, 0.f};
    // the old entries' key side (KPASS_OLD passes) and value rows (XR row
    // passes); a pass past the L old entries (uniform) is not loaded, so the
    // bounds above 8 entries cost nothing at short logs.  Pass 0 always
    // loads (a clamped, valid entry when L = 0).
    Raw klog[KPASS_OLD];
    float glog_s[KPASS_OLD];
    f4 glog4[KPASS_OLD];
    RawX xrow[XR];
    {
        const size_t el = (size_t)n * C + last;
        if (GDN)
            glast_s = p.logG[el];
        else
            glast4 = *reinterpret_cast<const f4 *>(p.logG + el * DK + c4);
#pragma unroll
        for (int ps = 0; ps < KPASS_OLD; ++ps) {
            if (ps > 0 && ps * EPP >= L) continue;
            const size_t e = (size_t)n * C + min(ps * EPP + ke, last);
            klog[ps] = *reinterpret_cast<const Raw *>(static_cast<const TIn *>(p.logK) + e * DK + c4);
            if (GDN)
                glog_s[ps] = p.logG[e];
            else
                glog4[ps] = *reinterpret_cast<const f4 *>(p.logG + e * DK + c4);
        }
        const TX *xin = static_cast<const TX *>(p.logX) + (size_t)n * C * DV + col0 + cq;
#pragma unroll
        for (int j = 0; j < XR; ++j)
            if (j == 0 || ESTEP * j < L) xrow[j] = *reinterpret_cast<const RawX *>(xin + (size_t)min(ebase + ESTEP * j, last) * DV);
    }
    // the small loads above all go out before the tile's (loads complete in
    // issue order, so one placed after the tile could only be used once the
    // whole tile has arrived; the matrix-core form uses the values early)
    if constexpr (MM) __builtin_amdgcn_sched_barrier(0);
    const size_t tile4 = (size_t)n * (DK * DV / 4) + (col0 + cq) / 4 + (size_t)rbase * (DV / 4);
    const f4 *src4 = reinterpret_cast<const f4 *>(p.base) + tile4;
    f4 s[R];
#pragma unroll
    for (int i = 0; i < R; ++i) s[i] = __builtin_nontemporal_load(src4 + (size_t)i * RSTEP * (DV / 4));
    // every load above is issued before anything consumes one (a consumer
    // scheduled among them would wait for all loads issued before it)
    __builtin_amdgcn_sched_barrier(0);
    // matrix-core form: the values go to LDS here so that they hold no registers
    // through phases B and C (every wave writes the same values; no branch, so
    // that no load is sunk past the tile)
    auto vrow = [&](int t) { return t > tf ? CMAX + t - tf - 1 : L + t; };
    auto stage_tokens = [&]() {
        if (DELTA) s_beta[(c4 == 0 && ke < K) ? ke : KM] = beta_t;
        if constexpr (MM) {
#pragma unroll
            for (int t = 0; t < KM; ++t) s_x[(t < K ? vrow(t) : CP) * TV + tid % TV] = to_f32(vraw[t]);
        }
    };
    stage_tokens();

    // One segment of the call.  The first may replay the old log; a later one
    // starts from an empty log, so its code (FIRST false) holds none of the
    // old entries' registers.
    auto run_segment = [&](auto first_tag) {
        constexpr bool FIRST = decltype(first_tag)::value;

        // ---------------- Phase B1: every token's inputs into LDS (group ke = token) ----------------
        const f4 kt_in = In4<TIn>::unpack(kraw);
        const f4 qt_in = In4<TIn>::unpack(qraw);
        if (ke < K) {
            *reinterpret_cast<f4 *>(&s_k[ke][c4]) = kt_in;
            *reinterpret_cast<f4 *>(&s_q[ke][c4]) = qt_in;
            if (GDN) {
                if (c4 == 0) s_lg[ke][0] = log2f(alpha);
            } else {
                *reinterpret_cast<f4 *>(&s_lg[ke][c4]) = log2v(dec4);
            }
        }
        if (ke == 0) {  // g_{-1} = g_L, newest old entry's cumulative log-decay
            if (GDN) {
                if (c4 == 0) s_g[0][0] = FIRST && L > 0 ? glast_s : 0.f;
            } else {
                *reinterpret_cast<f4 *>(&s_g[0][c4]) = FIRST && L > 0 ? glast4 : f4{0.f, 0.f, 0.f, 0.f};
            }
        }
        __syncthreads();
        // prefix sums of the log-decays: g_t for every token (group 0, four
        // channels per thread); a token past the fold also gets g'_t, its sum
        // from the fold, in place of its own log-decay
        if (ke == 0) {
            if (GDN) {
                if (c4 == 0) {
                    float g = s_g[0][0], g2 = 0.f;
                    for (int t = 0; t < K; ++t) {
                        const float lg = s_lg[t][0];
                        g += lg;
                        s_g[t + 1][0] = g;
                        if (!SEG && t > tf) {
                            g2 += lg;
                            s_lg[t][0] = g2;
                        }
                    }
                }
            } else {
                f4 g = *reinterpret_cast<const f4 *>(&s_g[0][c4]), g2 = {0.f, 0.f, 0.f, 0.f};
                for (int t = 0; t < K; ++t) {
                    const f4 lg = *reinterpret_cast<const f4 *>(&s_lg[t][c4]);
                    g += lg;
                    *reinterpret_cast<f4 *>(&s_g[t + 1][c4]) = g;
                    if (!SEG && t > tf) {
                        g2 += lg;
                        *reinterpret_cast<f4 *>(&s_lg[t][c4]) = g2;
                    }
                }
            }
        }
        __syncthreads();

        auto g_at = [&](int idx) -> f4 {  // g_{idx-1} for the thread's four channels
            if (GDN) {
                const float g = s_g[idx][0];
                return f4{g, g, g, g};
            }
            return *reinterpret_cast<const f4 *>(&s_g[idx][c4]);
        };

        // ---------------- Phase B2: per token: scaled key / query, dot, log append ----------------
        {
            // every group reduces its (valid, clamped) token's dot so that the lane
            // exchanges run with the whole wave active
            float part;
            if (DELTA)
                part = dot4(kt_in, qt_in);
            else
                part = dot4(qt_in * bon4, kt_in);
            part = group_sum_valu<KL>(part);
            if (ke < K && c4 == 0) s_dot[ke] = part;
        }
        if (ke < K) {
            const int t = ke;
            const f4 rho = DELTA ? g_at(t + 1) : g_at(t);
            const f4 sc = exp2v(rho);
            const f4 m0 = sc * kt_in, m1 = sc * qt_in;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int at = mv_at(c4 + c);
                if (DELTA) s_mv0[t][at] = m0[c];
                s_mv1[t][at] = m1[c];
            }
            if (!fold && tile == 0) {  // entry L + t of the log: the key copy and its log-decay
                const size_t e = (size_t)n * C + L + t;
                *reinterpret_cast<Raw *>(static_cast<TIn *>(p.logK) + e * DK + c4) = kraw;
                if (GDN) {
                    if (c4 == 0) p.logG[e] = g_at(t + 1).x;
                } else {
                    *reinterpret_cast<f4 *>(p.logG + e * DK + c4) = g_at(t + 1);
                }
            }
        }
        if (fold && ke == 0) *reinterpret_cast<f4 *>(&s_scale[c4]) = exp2v(g_at(SEG ? K : tf + 1));

        // ---------------- Phase B3: coefficients of every (token, entry) pair ----------------
        const f4 gend = g_at(SEG ? K : tf + 1);  // g_f: the fold's decay point
#pragma unroll
        for (int ps = 0; ps < KPASS; ++ps) {
            if (ps > 0 && ps * EPP >= NE) break;
            const int e = ps * EPP + ke;
            const int po = ps < KPASS_OLD ? ps : KPASS_OLD - 1;
            const bool is_old = FIRST && ps < KPASS_OLD && e < L;
            const bool is_new = e >= L && e < NE;
            f4 ke4, ge4;
            if (is_old) {
                ke4 = In4<TIn>::unpack(klog[po]);
                ge4 = GDN ? f4{glog_s[po], glog_s[po], glog_s[po], glog_s[po]} : glog4[po];
            } else if (is_new) {
                ke4 = *reinterpret_cast<const f4 *>(&s_k[e - L][c4]);
                ge4 = g_at(e - L + 1);
            } else {
                ke4 = f4{0.f, 0.f, 0.f, 0.f};
                ge4 = f4{0.f, 0.f, 0.f, 0.f};
            }
            // every token's partial dots first, then one batch of lane reductions
            float pk[KM], pq[KM];
#pragma unroll
            for (int t = 0; t < KM; ++t) {
                pk[t] = 0.f;
                pq[t] = 0.f;
                if (t < K && (is_old || (is_new && e - L < t))) {
                    const f4 rho = DELTA ? g_at(t + 1) : g_at(t);
                    const f4 kt = ke4 * exp2v(rho - ge4);
                    if (DELTA) pk[t] = dot4(kt, *reinterpret_cast<const f4 *>(&s_k[t][c4]));
                    pq[t] = dot4(kt, *reinterpret_cast<const f4 *>(&s_q[t][c4]));
                }
            }
            // in batches of four tokens, so that the independent exchanges of a
            // batch interleave; the second batch only when the chunk reaches it
            // (RWKV6 needs no key-side coefficients)
#pragma unroll
            for (int h = 0; h < KM; h += 4) {
                if (h > 0 && K <= h) break;
#pragma unroll
                for (int t = h; t < h + 4; ++t) {
                    if (DELTA) pk[t] = group_sum_valu<KL>(pk[t]);
                    pq[t] = group_sum_valu<KL>(pq[t]);
                }
            }
            if (c4 == 0 && e < NE) {
#pragma unroll
                for (int t = 0; t < KM; ++t) {
                    if (t < K) {
                        if (DELTA) s_coef[0][t][e] = pk[t];
                        s_coef[ZS][t][e] = pq[t];
                    }
                }
            }
            if (fold && (is_old || is_new) && (SEG || e < C))
                *reinterpret_cast<f4 *>(&s_kt[e * DK + c4]) = ke4 * exp2v(gend - ge4);
        }
        if constexpr (!SEG) {
            // The tokens past a fold start the new log: group j writes entry j,
            // token f + 1 + j's key copy (its input bits, from the exact fp32
            // copy) and g'_j.  Slot j is the one whose old entry this same group
            // read in phase A (or a slot no group read), and the group has used
            // that entry above, so the write cannot overtake the read.
            const int t = tf + 1 + ke;
            if (fold && t < K && tile == 0) {
                const size_t e = (size_t)n * C + ke;
                *reinterpret_cast<Raw *>(static_cast<TIn *>(p.logK) + e * DK + c4) =
                    Pack4<TIn>::pack(*reinterpret_cast<const f4 *>(&s_k[t][c4]));
                if (GDN) {
                    if (c4 == 0) p.logG[e] = s_lg[t][0];
                } else {
                    *reinterpret_cast<f4 *>(p.logG + e * DK + c4) = *reinterpret_cast<const f4 *>(&s_lg[t][c4]);
                }
            }
        }
        if (fold) {
            // old value factors of the tile for the fold; zero the fold's entry
            // slots from C up to a multiple of four
#pragma unroll
            for (int j = 0; j < XR; ++j) {
                const int i = ebase + ESTEP * j;
                if (FIRST && i < L) *reinterpret_cast<f4 *>(&s_x[i * TV + cq]) = In4<TX>::unpack(xrow[j]);
            }
            constexpr int W = DK > TV ? DK : TV;
            const int pad = ((C + 3) & ~3) - C;
            for (int idx = tid; idx < pad * W; idx += NT) {
                const int i = C + idx / W;
                const int c = idx % W;
                if (c < DK) s_kt[i * DK + c] = 0.f;
                if (c < TV) s_x[i * TV + c] = 0.f;
            }
        }
        __syncthreads();


        // ---------------- Phase C: base products of every token from the register tile ----------------
        if constexpr (MM) {
            // On the matrix cores: P[m][col] = sum_row A[m][row] S[row][col] over this
            // wave's rows, with the 16 vectors m = (side, token) = (m / 8, m % 8):
            // side 0 the scaled keys, side 1 the scaled queries (receptances).  The
            // register tile already has the 16x16x4 operand layout: in k-step i,
            // lane l holds row rbase + RSTEP i (rbase = its wave's first row + l/16)
            // and columns cq + c (cq = its wave's first column + 4 (l % 16)), so
            // component c of s[i] is the B operand of the c-th product, and lane l
            // supplies A[l % 16][that row].  The old log joins as XR more k-steps
            // with the replay coefficients as A and the logged value rows as B.
            typedef float m4 __attribute__((ext_vector_type(4)));
            const int m = lane & 15;
            const int kr = lane >> 4;
            const int side = m >> 3, tm = m & 7;
            // RWKV6 has only the query side: its key-side vectors are zero
            const bool live = tm < K && (DELTA || side == 1);
            const float *mv = (side || !DELTA) ? &s_mv1[tm][0] : &s_mv0[tm][0];
            float a[R];
#pragma unroll
            for (int i4 = 0; i4 < R / 4; ++i4) {
                const f4 v = *reinterpret_cast<const f4 *>(&mv[mv_at(rbase) + 4 * i4]);
#pragma unroll
                for (int c = 0; c < 4; ++c) a[4 * i4 + c] = live ? v[c] : 0.f;
            }
            // the products below are written over the scaled vectors
            __syncthreads();
            m4 acc[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] = m4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < R; ++i) {
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], s[i][c], acc[c], 0, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < XR; ++j) {
                if (j > 0 && ESTEP * j >= L) continue;  // a row pass with no old entry (not loaded)
                // entries at or past L were loaded from a clamped index and may be
                // anything (an unused slot holds whatever the workspace held): zero
                // both operands, since 0 * NaN would poison the sum
                const int e = ebase + ESTEP * j;
                const float co = (FIRST && live && e < L) ? s_coef[DELTA ? side : ZS][tm][e] : 0.f;
                const f4 xv = FIRST && e < L ? In4<TX>::unpack(xrow[j]) : f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(co, xv[c], acc[c], 0, 0, 0);
            }
            // lane l holds P[4 (l / 16) + q][cq + c] in acc[c][q]
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int mo = 4 * kr + q;
                if (DELTA || (mo >> 3) == 1)
                    *reinterpret_cast<f4 *>(&s_red[mo & 7][rblk][DELTA ? (mo >> 3) : 0][cq]) =
                        f4{acc[0][q], acc[1][q], acc[2][q], acc[3][q]};
            }
        } else {
#pragma unroll
            for (int t = 0; t < KM; ++t) {
                if (t >= K) break;
                f4 y = {0.f, 0.f, 0.f, 0.f}, z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i4 = 0; i4 < R / 4; ++i4) {
                    const f4 a = DELTA ? *reinterpret_cast<const f4 *>(&s_mv0[t][mv_at(rbase) + 4 * i4]) : f4{0.f, 0.f, 0.f, 0.f};
                    const f4 b = *reinterpret_cast<const f4 *>(&s_mv1[t][mv_at(rbase) + 4 * i4]);
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        if (DELTA) y += s[4 * i4 + c] * a[c];
                        z += s[4 * i4 + c] * b[c];
                    }
                }
#pragma unroll
                for (int j = 0; j < XR; ++j) {
                    const int i = ebase + ESTEP * j;
                    if (FIRST && i < L) {
                        const f4 x = In4<TX>::unpack(xrow[j]);
                        if (DELTA) y += s_coef[0][t][i] * x;
                        z += s_coef[ZS][t][i] * x;
                    }
                }
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if (DELTA) y[c] = column_sum_valu<LPR>(y[c]);
                    z[c] = column_sum_valu<LPR>(z[c]);
                }
                if (lane < LPR) {
                    if (DELTA) *reinterpret_cast<f4 *>(&s_red[t][rblk][0][cq]) = y;
                    *reinterpret_cast<f4 *>(&s_red[t][rblk][ZS][cq]) = z;
                }
            }
        }
        __syncthreads();

        // ---------------- Phase D: per column, the chunk's tokens in order ----------------
        if (tid < TV) {
            const int jt = tid;
            const int j = col0 + jt;
            float xs[KM];  // value factors of the chunk's tokens in this column
#pragma unroll
            for (int t = 0; t < KM; ++t) {
                if (t >= K) break;
                float yj = 0.f, zj = 0.f;
#pragma unroll
                for (int w = 0; w < NWR; ++w) {
                    if (DELTA) yj += s_red[t][w][0][jt];
                    zj += s_red[t][w][ZS][jt];
                }
#pragma unroll
                for (int m = 0; m < KM; ++m) {
                    if (m >= t) break;
                    if (DELTA) yj += s_coef[0][t][L + m] * xs[m];
                    zj += s_coef[ZS][t][L + m] * xs[m];
                }
                const float vj = MM ? s_x[vrow(t) * TV + jt] : to_f32(vraw[t]);
                float xnew, o;
                if (DELTA) {
                    xnew = s_beta[t] * (vj - yj);
                    o = zj + s_dot[t] * xnew;
                } else {
                    xnew = vj;
                    o = zj + s_dot[t] * vj;
                }
                xs[t] = xnew;
                p.out[tb + t][(size_t)n * DV + j] = o;
                const bool past = !SEG && fold && t > tf;
                if (fold && !past) {
                    s_x[(L + t) * TV + jt] = xnew;
                } else {
                    // the old value rows this overwrites past a fold were
                    // consumed before phase C's barrier
                    const size_t e = (size_t)n * C + (past ? t - tf - 1 : L + t);
                    if (DELTA)
                        static_cast<float *>(p.logX)[e * DV + j] = xnew;
                    else
                        store_raw(static_cast<TIn *>(p.logX) + e * DV + j, vj);
                }
            }
        }

        // ---------------- Phase E: fold the log's C entries into the base when the chunk fills it ----------------
        if (fold) {
            __syncthreads();
            f4 *dst4 = reinterpret_cast<f4 *>(p.base) + tile4;
            if constexpr (MM) {
                // The rank-NE update on the matrix cores.  For row group g and
                // column offset c: P[M][n] = sum_e kt[e][row(M)] x[e][4 n + c] (columns
                // from the wave's first) with row(M) = the wave's first row + M / 4 +
                // RSTEP (4 g + M % 4), so that lane l ends with P[4 (l / 16) + q][l % 16]
                // = the update of its own s[4 g + q][c].  Each group's rows are stored
                // as soon as they are done, so that one group's products are live at
                // a time.
                // The entry slots from C up to a multiple of four are zero.
                typedef float m4 __attribute__((ext_vector_type(4)));
                const int m = lane & 15, kr = lane >> 4;
#pragma unroll
                for (int g = 0; g < R / 4; ++g) {
                    const int arow = rbase - kr + (m >> 2) + RSTEP * (4 * g + (m & 3));
                    m4 pc[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c) pc[c] = m4{0.f, 0.f, 0.f, 0.f};
                    for (int e = 0; e < C; e += 4) {
                        const float av = s_kt[(e + kr) * DK + arow];
                        const f4 bv = *reinterpret_cast<const f4 *>(&s_x[(e + kr) * TV + cq]);
#pragma unroll
                        for (int c = 0; c < 4; ++c) pc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv[c], pc[c], 0, 0, 0);
                    }
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int i = 4 * g + q;
                        const f4 o = s[i] * s_scale[rbase + RSTEP * i] + f4{pc[0][q], pc[1][q], pc[2][q], pc[3][q]};
                        __builtin_nontemporal_store(o, dst4 + (size_t)i * RSTEP * (DV / 4));
                        if constexpr (SEG) s[i] = o;
                    }
                }
            } else {
                f4 acc[R];
#pragma unroll
                for (int i = 0; i < R; ++i) acc[i] = s[i] * s_scale[rbase + RSTEP * i];
                for (int e = 0; e < C; e += 4) {
                    const f4 x0 = *reinterpret_cast<const f4 *>(&s_x[(e + 0) * TV + cq]);
                    const f4 x1 = *reinterpret_cast<const f4 *>(&s_x[(e + 1) * TV + cq]);
                    const f4 x2 = *reinterpret_cast<const f4 *>(&s_x[(e + 2) * TV + cq]);
                    const f4 x3 = *reinterpret_cast<const f4 *>(&s_x[(e + 3) * TV + cq]);
#pragma unroll
                    for (int i = 0; i < R; ++i) {
                        const int row = rbase + RSTEP * i;
                        acc[i] += s_kt[(e + 0) * DK + row] * x0 + s_kt[(e + 1) * DK + row] * x1 +
                                  s_kt[(e + 2) * DK + row] * x2 + s_kt[(e + 3) * DK + row] * x3;
                    }
                }
#pragma unroll
                for (int i = 0; i < R; ++i) __builtin_nontemporal_store(acc[i], dst4 + (size_t)i * RSTEP * (DV / 4));
                if constexpr (SEG) {
#pragma unroll
                    for (int i = 0; i < R; ++i) s[i] = acc[i];
                }
            }
        }

    };
    run_segment(std::true_type{});
    if constexpr (SEG) {
        // the next segments: the rest of the call's tokens, each on an empty
        // log from the base the fold left in registers
        for (;;) {
            tb += K;
            if (tb >= p.K) break;
            L = 0;
            K = min(p.K - tb, C);
            fold = K == C;
            NE = K;
            tf = K - 1;
            __syncthreads();  // every read of the last segment's LDS is done
            load_tokens();
            stage_tokens();
            run_segment(std::false_type{});
        }
    }
}

// Tile shape of the chunk kernel: one workgroup per head.  The matrix-core
// form holds a square head of 128 or 64 over 2 DK threads (sixteen float4
// each at 128 x 128, eight at 64 x 64).  The vector form holds eight float4
// per thread where the head allows it (four at 32 x 32, 64 x 32 and
// 128 x 32), with at least one key-side group of lanes per token (2 DK
// threads) and one thread per value column: 16 KB over 128 threads at
// 64 x 64, 4 KB over 64 at 32 x 32.
template <int DK, int DV>
struct ChunkShape {
    static constexpr bool CAN_MM = DK == DV && (DK == 128 || DK == 64);
    static constexpr int TV = DV;
    static constexpr int A = 2 * DK > DV ? 2 * DK : DV;
    static constexpr int B = DK * DV / 32 > 64 ? DK * DV / 32 : 64;
    static constexpr int NT_VEC = A > B ? A : B;
    static constexpr int NT_MM = 2 * DK;
    // The fewest tokens per call that take the matrix-core form, which forms
    // all 16 product vectors whatever the call's K while the vector form's
    // work grows with K.  Measured on MI355X (RWKV6 B=128 H=32 d=64, C=8,
    // us/token, vector -> matrix cores): K=2 10.0 -> 11.1, K=3 7.8 -> 8.2,
    // K=4 6.3 -> 6.4, K=5 6.13 -> 6.05, K=6 5.5 -> 5.3, K=8 4.6 -> 4.1.  At
    // 128 x 128 the matrix cores win from two tokens on (a single token goes
    // to the single-token kernel), so the vector form is not built there.
    static constexpr int MM_FROM = DK == 128 ? 1 : 5;
};

template <int OP, typename TIn, int DK, int DV, int CMAX, bool SEG>
hipError_t launch_chunk_form(const ChunkParams &p, hipStream_t s) {
    using S = ChunkShape<DK, DV>;
    const unsigned blocks = (unsigned)p.N;
    if constexpr (S::CAN_MM) {
        if (p.K >= S::MM_FROM) {
            hipLaunchKernelGGL((chunk_kernel<OP, TIn, DK, DV, S::TV, S::NT_MM, CMAX, true, SEG>), dim3(blocks),
                               dim3(S::NT_MM), 0, s, p);
            return hipGetLastError();
        }
    }
    if constexpr (S::MM_FROM > 1 || !S::CAN_MM) {
        hipLaunchKernelGGL((chunk_kernel<OP, TIn, DK, DV, S::TV, S::NT_VEC, CMAX, false, SEG>), dim3(blocks),
                           dim3(S::NT_VEC), 0, s, p);
        return hipGetLastError();
    }
    return hipErrorInvalidValue;
}

template <int OP, typename TIn, int DK, int DV, int CMAX>
hipError_t launch_chunk_one(const ChunkParams &p, hipStream_t s) {
    if (!p.segmented) return launch_chunk_form<OP, TIn, DK, DV, CMAX, false>(p, s);
    // more tokens than C: C < KMAX_TOKENS, within the smallest bound
    if constexpr (CMAX == 8) return launch_chunk_form<OP, TIn, DK, DV, CMAX, true>(p, s);
    return hipErrorInvalidValue;
}

template <int OP, typename TIn, int DK, int DV>
hipError_t launch_chunk_bounded(int cmax, const ChunkParams &p, hipStream_t s) {
    if (cmax <= 8) return launch_chunk_one<OP, TIn, DK, DV, 8>(p, s);
    if (cmax <= 16) return launch_chunk_one<OP, TIn, DK, DV, 16>(p, s);
    return launch_chunk_one<OP, TIn, DK, DV, 32>(p, s);
}

template <int OP, typename TIn, int DK>
hipError_t launch_chunk_value_width(int DV, int cmax, const ChunkParams &p, hipStream_t s) {
    switch (DV) {
        case 32: return launch_chunk_bounded<OP, TIn, DK, 32>(cmax, p, s);
        case 64: return launch_chunk_bounded<OP, TIn, DK, 64>(cmax, p, s);
        case 128: return launch_chunk_bounded<OP, TIn, DK, 128>(cmax, p, s);
        default: return hipErrorInvalidValue;
    }
}

template <int OP, int DK>
hipError_t launch_chunk(int in_bf16, int DV, int cmax, const ChunkParams &p, hipStream_t s) {
    return in_bf16 ? launch_chunk_value_width<OP, bf16_bits, DK>(DV, cmax, p, s)
                   : launch_chunk_value_width<OP, float, DK>(DV, cmax, p, s);
}

}  // namespace dlk
