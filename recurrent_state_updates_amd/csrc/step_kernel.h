// step_kernel.h -- the decode-step kernel family for gfx950.
//
// One workgroup owns a D x TV tile of one head's fp32 state: all D key rows
// and TV of the D value columns (the pages' value-tile parallelism).  Its
// threads stream the tile once from HBM with coalesced 16-byte loads (a tile
// row is TV/4 lanes wide), keep it in registers, and do everything else
// around that single pass:
//
//   APPEND  o_t from base + log replay, new factor appended (base read only)
//   MERGE   the same token, then the rank-C fold of the whole log into the
//           base from registers (base read once, written once)
//   EAGER   the dense recurrence directly (base read once, written once)
//   FOLD    base + log written to a destination (merge / materialise)
//
// The method (DeltaLog; gist.science summary, sections "Meccanismo Core" and
// "Implementazione del Kernel"): the state is split along the value width;
// each work unit owns a base slice and its value-side log shard, and the
// key-side factors and log-decay metadata are shared by the tiles.  The
// pages run the key-side replay preparation as a separate stage once per
// slot-head; here every workgroup recomputes it in its prologue, from LDS,
// while its base loads are in flight -- a few hundred FLOPs per head against
// a 32 KB stream, cheaper than a second launch -- and the two tiles of a head
// run on the same XCD so the second reads the key-side log from L2.
//
// Algebra, per head, with cumulative base-2 log-decays g (reset at a fold):
//   logical state   S_L = diag(2^{g_L}) Sbar + sum_{i<L} diag(2^{g_L-g_i}) k_i x_i^T
//   delta rules     gn = g_L + log2(decay_t); khat = 2^{gn} k_t, qhat = 2^{gn} q_t
//                   y = Sbar^T khat + sum_i x_i <k_i 2^{gn-g_i}, k_t>
//                   z = Sbar^T qhat + sum_i x_i <k_i 2^{gn-g_i}, q_t>
//                   u_t = beta (v_t - y);  o_t = z + <k_t, q_t> u_t
//   RWKV6           rhat = 2^{g_L} r_t;  s = sum_c r u k
//                   o_t = Sbar^T rhat + sum_i v_i <k_i 2^{g_L-g_i}, r_t> + s v_t
//                   entry: (k_t, v_t, g_L + log2 w_t)
// A fold writes S = diag(2^{g}) Sbar + sum_i (k_i 2^{g-g_i}) x_i^T with g the
// decay point of the state being written.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "launch.h"

namespace dlk {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_bits;  // bfloat16 stored as its raw bits

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_bits b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Thread geometry of one workgroup over a D x TV tile (all D key rows, TV of
// the D value columns) of one head's state.
template <int D, int TV, int NT>
struct Geom {
    static constexpr int NTILE = D / TV;         // value tiles per head
    static constexpr int LPR = TV / 4;           // lanes per tile row (one float4 each)
    static constexpr int RPP = NT / LPR;         // rows per pass of the workgroup
    static constexpr int R = D / RPP;            // rows held by each thread
    static constexpr int NW = NT / 64;           // waves
    static constexpr int LPE = D < 64 ? D : 64;  // lanes per log entry in the key-side pass
    static constexpr int EPW = 64 / LPE;         // log entries per wave and round
    static constexpr int CPL = D / LPE;          // key channels per lane
    static_assert(D % TV == 0 && TV % 4 == 0 && NT % 64 == 0, "geometry");
    static_assert(NT % LPR == 0 && D % RPP == 0 && R >= 1, "the tile must divide evenly");
    static_assert(TV <= NT, "one thread per value column in the column stage");
};

// Tile shape per head width: 32 KB (D = 128, two value tiles per head),
// 16 KB (D = 64) and 4 KB (D = 32) per workgroup.
template <int D>
struct Shape {
    static constexpr int TV = D == 128 ? 64 : D;
    static constexpr int NT = D == 128 ? 256 : (D == 64 ? 128 : 64);
};

// Workgroups are handed to the eight XCDs round-robin in dispatch order.
// Map block b to (head, value tile) so that the tiles of one head are eight
// blocks apart -- on the same XCD, where the second reads the head's shared
// key-side log from that XCD's L2.
__device__ __forceinline__ void block_to_tile(int b, int N, int ntile, int &n, int &tile) {
    const int group = b / (8 * ntile);
    const int within = b - group * 8 * ntile;
    const int gs = min(8, N - group * 8);  // heads in this group (fewer in the last one)
    tile = within / gs;
    n = group * 8 + within % gs;
}

// Sum over aligned groups of W consecutive lanes.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int off = W / 2; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

template <int OP, typename TIn, int D, int TV, int NT, int MODE, int CMAX>
__global__ __launch_bounds__(NT) void step_kernel(const StepParams p) {
    using G = Geom<D, TV, NT>;
    constexpr int NTILE = G::NTILE, LPR = G::LPR, RPP = G::RPP, R = G::R, NW = G::NW;
    constexpr int LPE = G::LPE, EPW = G::EPW, CPL = G::CPL;
    constexpr bool DELTA = OP != OP_RWKV6;
    constexpr bool LOGGED = MODE != MODE_EAGER;  // reads a log
    constexpr bool TOKEN = MODE != MODE_FOLD;    // decodes a token
    constexpr bool WRITES = MODE != MODE_APPEND; // writes a dense state
    constexpr bool CUR_IN_LOG = MODE == MODE_MERGE && DELTA;  // fold the token as entry L
    constexpr int CP = LOGGED ? CMAX : 4;        // entry slots in LDS (multiple of 4)
    constexpr int KROUNDS = LOGGED ? (CMAX + NW * EPW - 1) / (NW * EPW) : 0;
    constexpr int XROUNDS = LOGGED ? (CMAX * TV + NT - 1) / NT : 0;
    using TX = typename std::conditional<DELTA, float, TIn>::type;  // value-side log dtype
    static_assert(CMAX % 4 == 0, "entry slots come in groups of four");

    __shared__ float s_mv0[D];     // khat (delta rules)
    __shared__ float s_mv1[D];     // qhat, or rhat (RWKV6)
    __shared__ float s_scale[D];   // factor on each base row when a state is written
    __shared__ float s_krow[D];    // current key, per row
    __shared__ float s_wrow[D];    // RWKV6: current decay, per row
    __shared__ __attribute__((aligned(16))) float s_ktT[LOGGED ? D * CP : 4];  // [row][entry]
    __shared__ __attribute__((aligned(16))) float s_x[LOGGED ? CP * TV : 4];   // [entry][tile col]
    __shared__ float s_coef[2][CP];  // replay coefficients: k side, q/r side
    __shared__ __attribute__((aligned(16))) float s_red[NW][2][TV];
    __shared__ __attribute__((aligned(16))) float s_u[TV];  // current value factor
    __shared__ float s_dot;          // <k,q> (delta rules) or sum r*bonus*k (RWKV6)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    int n, tile;
    block_to_tile(blockIdx.x, p.N, NTILE, n, tile);
    const int L = LOGGED ? p.L : 0;
    const int C = p.C;
    const int cg = tid % LPR;  // float4 column group: tile columns 4cg .. 4cg+3
    const int rs = tid / LPR;  // rows rs + RPP*i, i < R
    const int col0 = tile * TV;  // first value column of the tile

    // 1. Issue the base tile loads first: they are nearly all of the traffic.
    //    Row r of the tile is TV/4 float4 at head offset r*D/4 + col0/4.
    const size_t tile4 = (size_t)n * (D * D / 4) + col0 / 4 + (size_t)rs * (D / 4) + cg;
    const f4 *src4 = reinterpret_cast<const f4 *>(p.base) + tile4;
    f4 s[R];
#pragma unroll
    for (int i = 0; i < R; ++i) s[i] = __builtin_nontemporal_load(src4 + (size_t)i * RPP * (D / 4));

    // 2. This lane's key channels c = lc + LPE*m: token inputs and log-decays.
    const int se = lane / LPE;
    const int lc = lane % LPE;
    const TIn *kin = static_cast<const TIn *>(p.k) + (size_t)n * D;
    const TIn *qin = static_cast<const TIn *>(p.q) + (size_t)n * D;
    float kc[CPL], qc[CPL], dc[CPL], gnew[CPL], gref[CPL];
    float alpha = 1.f, glast = 0.f;
    if (OP == OP_GDN) {
        if (TOKEN) alpha = p.decay[n];
        if (LOGGED && L > 0) glast = p.logG[(size_t)n * C + (L - 1)];
    }
#pragma unroll
    for (int m = 0; m < CPL; ++m) {
        const int c = lc + LPE * m;
        kc[m] = 0.f;
        qc[m] = 0.f;
        dc[m] = 1.f;
        if (TOKEN) {
            kc[m] = to_f32(kin[c]);
            qc[m] = to_f32(qin[c]);
            dc[m] = (OP == OP_GDN) ? alpha : p.decay[(size_t)n * D + c];
        }
        float gl = glast;
        if (OP != OP_GDN && LOGGED && L > 0) gl = p.logG[((size_t)n * C + (L - 1)) * D + c];
        gnew[m] = gl + ((TOKEN && LOGGED) ? log2f(dc[m]) : 0.f);
        gref[m] = (DELTA && TOKEN) ? gnew[m] : gl;
    }

    // Per-row factors, the current entry and the append of the key side
    // (one writer per channel).
    if (wave == 0 && se == 0) {
#pragma unroll
        for (int m = 0; m < CPL; ++m) {
            const int c = lc + LPE * m;
            float sc;
            if (MODE == MODE_EAGER) {
                sc = dc[m];
                s_mv0[c] = dc[m] * kc[m];
                s_mv1[c] = DELTA ? dc[m] * qc[m] : qc[m];  // RWKV6 reads the pre-update state
            } else {
                sc = exp2f(gref[m]);
                s_mv0[c] = sc * kc[m];
                s_mv1[c] = sc * qc[m];
            }
            s_scale[c] = sc;
            s_krow[c] = kc[m];
            s_wrow[c] = dc[m];
            if (LOGGED && CUR_IN_LOG) s_ktT[c * CP + L] = kc[m];
            if (MODE == MODE_APPEND && tile == 0) {
                const size_t e = (size_t)n * C + L;
                static_cast<TIn *>(p.logK)[e * D + c] = kin[c];
                if (OP != OP_GDN) p.logG[e * D + c] = gnew[m];
            }
        }
        if (MODE == MODE_APPEND && OP == OP_GDN && tile == 0 && lane == 0)
            p.logG[(size_t)n * C + L] = gnew[0];
    }
    if (TOKEN && wave == 0) {
        float part = 0.f;
        if (se == 0) {
#pragma unroll
            for (int m = 0; m < CPL; ++m) {
                const int c = lc + LPE * m;
                part += DELTA ? kc[m] * qc[m] : qc[m] * p.bonus[(size_t)(n % p.H) * D + c] * kc[m];
            }
        }
        part = group_sum<64>(part);
        if (lane == 0) s_dot = part;
    }

    if (LOGGED) {
        // Key side of the log: decayed keys into LDS and, for a token, the
        // replay coefficients <k_i 2^{g-g_i}, k_t> and <k_i 2^{g-g_i}, q_t>.
#pragma unroll
        for (int r = 0; r < KROUNDS; ++r) {
            const int i0 = (r * NW + wave) * EPW;  // wave-uniform
            const int i = i0 + se;
            const bool valid = i < L;
            float pk = 0.f, pq = 0.f;
#pragma unroll
            for (int m = 0; m < CPL; ++m) {
                const int c = lc + LPE * m;
                if (valid) {
                    const size_t e = (size_t)n * C + i;
                    const float kv = to_f32(static_cast<const TIn *>(p.logK)[e * D + c]);
                    const float gi = (OP == OP_GDN) ? p.logG[e] : p.logG[e * D + c];
                    const float kt = kv * exp2f(gref[m] - gi);
                    s_ktT[c * CP + i] = kt;
                    pk += kt * kc[m];
                    pq += kt * qc[m];
                }
            }
            if (TOKEN && i0 < L) {
                pk = group_sum<LPE>(pk);
                pq = group_sum<LPE>(pq);
                if (valid && lc == 0) {
                    s_coef[0][i] = pk;
                    s_coef[1][i] = pq;
                }
            }
        }
        // Value side of the log: this tile's columns of entries 0..L-1.
        const TX *xin = static_cast<const TX *>(p.logX) + (size_t)n * C * D + col0;
#pragma unroll
        for (int r = 0; r < XROUNDS; ++r) {
            const int idx = tid + NT * r;
            if (idx < L * TV) s_x[idx] = to_f32(xin[(size_t)(idx / TV) * D + idx % TV]);
        }
        // Zero the slots between the last folded entry and the next multiple of four.
        if (WRITES) {
            const int ne = CUR_IN_LOG ? L + 1 : L;
            const int pad = ((ne + 3) & ~3) - ne;
            for (int idx = tid; idx < pad * D; idx += NT) {
                const int i = ne + idx / D;
                const int c = idx % D;
                s_ktT[c * CP + i] = 0.f;
                if (c < TV) s_x[i * TV + c] = 0.f;
            }
        }
    }
    __syncthreads();

    if (TOKEN) {
        // 3. Matrix-vector products against the base tile held in registers.
        f4 y = {0.f, 0.f, 0.f, 0.f}, z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int row = rs + RPP * i;
            if (DELTA) y += s[i] * s_mv0[row];
            z += s[i] * s_mv1[row];
        }
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) {
            if (DELTA) {
                y.x += __shfl_xor(y.x, off);
                y.y += __shfl_xor(y.y, off);
                y.z += __shfl_xor(y.z, off);
                y.w += __shfl_xor(y.w, off);
            }
            z.x += __shfl_xor(z.x, off);
            z.y += __shfl_xor(z.y, off);
            z.z += __shfl_xor(z.z, off);
            z.w += __shfl_xor(z.w, off);
        }
        if (lane < LPR) {
            if (DELTA) *reinterpret_cast<f4 *>(&s_red[wave][0][4 * cg]) = y;
            *reinterpret_cast<f4 *>(&s_red[wave][1][4 * cg]) = z;
        }
        __syncthreads();

        // 4. Column stage: one thread per value column of the tile.
        if (tid < TV) {
            const int jt = tid;        // column within the tile
            const int j = col0 + jt;   // column within the head
            float yj = 0.f, zj = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                if (DELTA) yj += s_red[w][0][jt];
                zj += s_red[w][1][jt];
            }
            if (LOGGED) {
                for (int i = 0; i < L; ++i) {
                    const float x = s_x[i * TV + jt];
                    if (DELTA) yj += s_coef[0][i] * x;
                    zj += s_coef[1][i] * x;
                }
            }
            const TIn vraw = static_cast<const TIn *>(p.v)[(size_t)n * D + j];
            const float vj = to_f32(vraw);
            float xnew, o;
            if (DELTA) {
                xnew = p.beta[n] * (vj - yj);
                o = zj + s_dot * xnew;
            } else {
                xnew = vj;
                o = zj + s_dot * vj;
            }
            p.out[(size_t)n * D + j] = o;
            if (MODE == MODE_APPEND) {
                const size_t e = (size_t)n * C + L;
                if (DELTA)
                    static_cast<float *>(p.logX)[e * D + j] = xnew;
                else
                    static_cast<TIn *>(p.logX)[e * D + j] = vraw;
            }
            if (LOGGED && CUR_IN_LOG)
                s_x[L * TV + jt] = xnew;
            else
                s_u[jt] = xnew;
        }
        if (WRITES) __syncthreads();
    }

    if (WRITES) {
        // 5. Write the state: row scale, rank-(entries) update from LDS, then
        //    the current token for RWKV6 and the eager form.
        const int ne = CUR_IN_LOG ? L + 1 : L;
        f4 acc[R];
#pragma unroll
        for (int i = 0; i < R; ++i) acc[i] = s[i] * s_scale[rs + RPP * i];
        if (LOGGED) {
            for (int e = 0; e < ne; e += 4) {
                const f4 x0 = *reinterpret_cast<const f4 *>(&s_x[(e + 0) * TV + 4 * cg]);
                const f4 x1 = *reinterpret_cast<const f4 *>(&s_x[(e + 1) * TV + 4 * cg]);
                const f4 x2 = *reinterpret_cast<const f4 *>(&s_x[(e + 2) * TV + 4 * cg]);
                const f4 x3 = *reinterpret_cast<const f4 *>(&s_x[(e + 3) * TV + 4 * cg]);
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    const f4 kt = *reinterpret_cast<const f4 *>(&s_ktT[(rs + RPP * i) * CP + e]);
                    acc[i] += kt.x * x0 + kt.y * x1 + kt.z * x2 + kt.w * x3;
                }
            }
        }
        if (TOKEN && !CUR_IN_LOG) {
            const f4 u = *reinterpret_cast<const f4 *>(&s_u[4 * cg]);
#pragma unroll
            for (int i = 0; i < R; ++i) {
                const int row = rs + RPP * i;
                if (MODE == MODE_MERGE)  // RWKV6: decay the logical state, then add k v^T
                    acc[i] = acc[i] * s_wrow[row] + s_krow[row] * u;
                else
                    acc[i] += s_krow[row] * u;
            }
        }
        f4 *dst4 = reinterpret_cast<f4 *>(p.dst) + tile4;
#pragma unroll
        for (int i = 0; i < R; ++i) __builtin_nontemporal_store(acc[i], dst4 + (size_t)i * RPP * (D / 4));
    }
}

template <int OP, typename TIn, int D, int MODE, int CMAX>
hipError_t launch_one(const StepParams &p, hipStream_t s) {
    constexpr int TV = Shape<D>::TV, NT = Shape<D>::NT;
    const unsigned blocks = (unsigned)p.N * (D / TV);
    hipLaunchKernelGGL((step_kernel<OP, TIn, D, TV, NT, MODE, CMAX>), dim3(blocks), dim3(NT), 0, s, p);
    return hipGetLastError();
}

template <int OP, typename TIn, int D>
hipError_t launch_mode(int mode, int cmax, const StepParams &p, hipStream_t s) {
    const bool small = cmax <= 8;
    switch (mode) {
        case MODE_APPEND:
            return small ? launch_one<OP, TIn, D, MODE_APPEND, 8>(p, s)
                         : launch_one<OP, TIn, D, MODE_APPEND, 32>(p, s);
        case MODE_MERGE:
            return small ? launch_one<OP, TIn, D, MODE_MERGE, 8>(p, s)
                         : launch_one<OP, TIn, D, MODE_MERGE, 32>(p, s);
        case MODE_FOLD:
            return small ? launch_one<OP, TIn, D, MODE_FOLD, 8>(p, s)
                         : launch_one<OP, TIn, D, MODE_FOLD, 32>(p, s);
        case MODE_EAGER:
            return launch_one<OP, TIn, D, MODE_EAGER, 4>(p, s);
        default:
            return hipErrorInvalidValue;
    }
}

template <int OP, typename TIn>
hipError_t launch_width(int D, int mode, int cmax, const StepParams &p, hipStream_t s) {
    switch (D) {
        case 32: return launch_mode<OP, TIn, 32>(mode, cmax, p, s);
        case 64: return launch_mode<OP, TIn, 64>(mode, cmax, p, s);
        case 128: return launch_mode<OP, TIn, 128>(mode, cmax, p, s);
        default: return hipErrorInvalidValue;
    }
}

template <int OP>
hipError_t launch_op(int in_bf16, int D, int mode, int cmax, const StepParams &p, hipStream_t s) {
    return in_bf16 ? launch_width<OP, bf16_bits>(D, mode, cmax, p, s)
                   : launch_width<OP, float>(D, mode, cmax, p, s);
}

}  // namespace dlk
