// step_kernel.h -- the decode-step kernel family for gfx950.
//
// One workgroup owns a DK x TV tile of one head's fp32 state: all DK key rows
// and TV of the DV value columns (the pages' value-tile parallelism; the
// single-token kernels use TV = DV, one tile per head, see Shape, except for
// the last heads of a 128 x 128 launch, which step_kernel_tail runs as two
// half-width tiles each).  Its
// threads stream the tile once from HBM with coalesced 16-byte loads (a tile
// row is TV/4 lanes wide), keep it in registers, and do everything else
// around that single pass:
//
//   APPEND  o_t from base + log replay, new factor appended (base read only)
//   MERGE   the same token, then the rank-C fold of the whole log into the
//           base from registers (base read once, written once)
//   EAGER   the dense recurrence directly (base read once, written once)
//   FOLD    base + log written to a destination (merge / materialise)
//   AUTO    per-slot logs: a slot's workgroups APPEND, or MERGE when this
//           token fills that slot's log
//   PREP / PREPPED  the two stages of the split-replay variant (below)
//
// The method (DeltaLog; gist.science summary, sections "Meccanismo Core" and
// "Implementazione del Kernel"): the state is split along the value width;
// each work unit owns a base slice and its value-side log shard, and the
// key-side factors and log-decay metadata are shared by the tiles.  The
// pages run the key-side replay preparation as a separate stage once per
// slot-head; here every workgroup recomputes it in its prologue, from
// registers, while its base loads are in flight -- a few hundred FLOPs per
// head against a 16-64 KB stream; with one tile per head nothing is
// recomputed, and with several (the chunk kernel) the tiles of a head run
// on the same XCD so the later ones read the key-side log from L2.  The pages' staged form
// is built too, for comparison: PREP runs that prologue once per head and
// stores its results in a small per-head record, and PREPPED is the append
// whose workgroups read the record instead.  On MI355X the staged form costs
// about 5 us more per append: its first stage is a serial, latency-bound
// launch.
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

typedef unsigned int u2 __attribute__((ext_vector_type(2)));  // four packed bfloat16

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_bits b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Four consecutive input elements, loaded as one 16-byte (fp32) or 8-byte
// (bf16) vector and unpacked to fp32.
template <typename TIn>
struct In4;
template <>
struct In4<float> {
    typedef f4 raw;
    __device__ static f4 unpack(f4 r) { return r; }
};
template <>
struct In4<bf16_bits> {
    typedef u2 raw;
    __device__ static f4 unpack(u2 r) {
        f4 o;
        o.x = __uint_as_float(r.x << 16);
        o.y = __uint_as_float(r.x & 0xffff0000u);
        o.z = __uint_as_float(r.y << 16);
        o.w = __uint_as_float(r.y & 0xffff0000u);
        return o;
    }
};

__device__ __forceinline__ float dot4(f4 a, f4 b) { return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w; }

__device__ __forceinline__ f4 exp2v(f4 a) {
    f4 o;
    o.x = exp2f(a.x);
    o.y = exp2f(a.y);
    o.z = exp2f(a.z);
    o.w = exp2f(a.w);
    return o;
}

__device__ __forceinline__ f4 log2v(f4 a) {
    f4 o;
    o.x = log2f(a.x);
    o.y = log2f(a.y);
    o.z = log2f(a.z);
    o.w = log2f(a.w);
    return o;
}

// Thread geometry of one workgroup over a DK x TV tile (all DK key rows, TV
// of the DV value columns) of one head's state.
template <int DK, int DV, int TV, int NT>
struct Geom {
    static constexpr int NTILE = DV / TV;  // value tiles per head
    static constexpr int LPR = TV / 4;     // lanes per tile row (one float4 each)
    static constexpr int RPP = NT / LPR;   // rows per pass of the workgroup
    static constexpr int R = DK / RPP;     // rows held by each thread
    static constexpr int NW = NT / 64;     // waves
    static constexpr int KL = DK / 4;      // key-side lanes per log entry (4 channels each)
    static constexpr int EPP = NT / KL;    // log entries per key-side pass
    static_assert(DV % TV == 0 && TV % 4 == 0 && NT % 64 == 0, "geometry");
    static_assert(NT % LPR == 0 && DK % RPP == 0 && R >= 1, "the tile must divide evenly");
    static_assert(TV <= NT && KL <= 64 && NT % KL == 0, "column stage and key-side groups");
};

// Tile shape of the single-token kernels: one workgroup per head at every
// width.  A thread holds eight float4 of the state (sixteen at 128 x 128),
// with at least one thread per value column for the column stage and one
// wave per workgroup: 64 KB over 256 threads at 128 x 128, 16 KB over 128 at
// 64 x 64, 4 KB over 64 (four float4 each) at 32 x 32; the rectangular heads
// between them take 64 to 256 threads of eight.  A whole head is one
// contiguous block, which streams about 7 % faster on MI355X than two
// 64-column halves of it (rows read as 256-byte pieces at a 512-byte
// stride), for the append and the fold alike.  At 128 x 128 the decode modes
// use 256 threads of sixteen float4 each: four heads per CU instead of
// three, appends 2-4 % faster than with 512 threads of eight.  The
// decode-and-fold keeps the append's shape, so that per-slot decode (one
// kernel that appends or folds per slot) adds its column sums in the same
// order as the lockstep kernels and gives the same bits.  At 128 x 128 the
// standalone fold and the eager kernel keep 512 threads, 1-2 % faster for
// them; the fold's result does not depend on the shape (no column sums).
template <int DK, int DV, int MODE>
struct Shape {
    static constexpr bool WIDE = MODE == MODE_FOLD || MODE == MODE_EAGER;
    static constexpr int TV = DV;
    static constexpr int EIGHT = DK * DV / 32;  // threads of eight float4 each
    static constexpr int BASE = EIGHT > 256 ? 256 : EIGHT;
    static constexpr int NT0 = BASE > DV ? BASE : DV;
    static constexpr int NT1 = NT0 > 64 ? NT0 : 64;
    static constexpr int NT = (DK == 128 && DV == 128 && WIDE) ? 512 : NT1;
};

// Workgroups are handed to the eight XCDs round-robin in dispatch order
// (block b runs on XCD b % 8).  With XCD set, block b is mapped so that each
// XCD walks one contiguous range of (head, tile) pairs in order, so each L2
// gathers whole contiguous lines of the outputs and log entries it writes
// instead of every eighth head's pieces.  Without it, block b is pair b and
// the chip sweeps the heads in order, all eight XCDs on neighbouring heads.
// Which is faster depends on the kernel, measured on MI355X (bench.py, back
// to back and cold): the contiguous ranges for the single-token kernels on
// 64 KB heads (GDN C=8 52.3 against 55.7 us/token, KDA 55.5 against 57.2);
// the dispatch order for 16 KB heads (RWKV6 C=8 15.5 against 16.4, a read of
// every 16 KB head 8.2 against 10.1 us) and for the multi-token kernel (GDN
// eight tokens per call 13.1 against 13.6 us/token, KDA 13.3 against 14.1,
// RWKV6 4.6 against 4.9).
template <bool XCD>
__device__ __forceinline__ void block_to_tile(int b, int N, int ntile, int &n, int &tile) {
    int g = b;
    if (XCD) {
        const int nb = N * ntile;
        const int x = b & 7, k = b >> 3;
        g = x * (nb >> 3) + min(x, nb & 7) + k;  // XCD x owns pairs [off_x, off_x + count_x)
    }
    n = g / ntile;
    tile = g - n * ntile;
}

// The single-token kernels (and the probes that bound them) map 64 KB heads
// in contiguous ranges per XCD and smaller heads in dispatch order.
template <int DK, int DV>
struct StepOrder {
    static constexpr bool XCD = DK * DV >= 128 * 128;
};

// Lane exchanges that stay in the VALU (no LDS round trip): DPP moves within
// rows of 16 lanes and the gfx950 permlane swaps across rows.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int DPP_XOR8 = 0x128;        // row_ror:8 (within a row of 16, a rotation by 8 is xor 8)
constexpr int DPP_HALF_MIRROR = 0x141; // lane i -> 7 - i within each group of 8
constexpr int DPP_MIRROR = 0x140;      // lane i -> 15 - i within each row

// x[l] + x[l ^ 16]: the swap returns the lane's even-row and odd-row values.
__device__ __forceinline__ float xor16_sum(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// x[l] + x[l ^ 32]: the swap returns the lane's low-half and high-half values.
__device__ __forceinline__ float xor32_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over aligned groups of W lanes.  Each step adds two values already equal
// across their sub-groups, so the mirrors act as exchanges between sub-groups
// and every lane of a group ends with the same bits.
template <int W>
__device__ __forceinline__ float group_sum_valu(float x) {
    static_assert(W == 1 || W == 2 || W == 4 || W == 8 || W == 16 || W == 32 || W == 64, "group width");
    if (W >= 2) x += dpp_mov<DPP_XOR1>(x);
    if (W >= 4) x += dpp_mov<DPP_XOR2>(x);
    if (W >= 8) x += dpp_mov<DPP_HALF_MIRROR>(x);
    if (W >= 16) x += dpp_mov<DPP_MIRROR>(x);
    if (W >= 32) x = xor16_sum(x);
    if (W >= 64) x = xor32_sum(x);
    return x;
}

// Sum over the lanes of a wave that share l % P (P = 8, 16 or 32 lanes per row
// of a tile): the partial products of one value column.
template <int P>
__device__ __forceinline__ float column_sum_valu(float x) {
    static_assert(P == 8 || P == 16 || P == 32 || P == 64, "lanes per tile row");
    if (P <= 8) x += dpp_mov<DPP_XOR8>(x);
    if (P <= 16) x = xor16_sum(x);
    if (P <= 32) x = xor32_sum(x);
    return x;
}

// Optional occupancy floor in waves per SIMD (0: the compiler's choice).  A
// floor that forces spills has been seen to place register copies inside a
// lane-masked branch (the value of only the active lanes is kept), so the
// default leaves the register budget to the compiler.
#ifndef DLK_MIN_WAVES
#define DLK_MIN_WAVES 0
#endif
#if DLK_MIN_WAVES > 0
#define DLK_OCCUPANCY __attribute__((amdgpu_waves_per_eu(DLK_MIN_WAVES, 8)))
#else
#define DLK_OCCUPANCY
#endif
//
// Structure: every global load the workgroup needs -- its base tile, the
// token's inputs, the log entries (at clamped, always valid indices, masked
// afterwards) and the value input of the column stage -- is issued first,
// with no branch and no dependence between them, so that one memory
// round-trip covers them all; only then does any arithmetic start.
template <int OP, typename TIn, int DK, int DV, int TV, int NT, int MODE, int CMAX>
__device__ __forceinline__ void step_body(const StepParams &p, const int n, const int tile) {
    using G = Geom<DK, DV, TV, NT>;
    constexpr int NTILE = G::NTILE, LPR = G::LPR, RPP = G::RPP, R = G::R, NW = G::NW;
    constexpr int KL = G::KL, EPP = G::EPP;
    constexpr bool GDN = OP == OP_GDN;
    constexpr bool DELTA = OP != OP_RWKV6;
    constexpr bool LOGGED = MODE != MODE_EAGER;  // reads a log
    constexpr bool TOKEN = MODE != MODE_FOLD;    // decodes a token
    constexpr bool AUTO = MODE == MODE_AUTO;     // append or fold, per slot, at run time
    constexpr bool PREP = MODE == MODE_PREP;     // split replay: key-side stage, no tile
    constexpr bool PREPPED = MODE == MODE_PREPPED;  // split replay: key side from the record
    constexpr bool CAN_WRITE =                   // may write a dense state
        MODE == MODE_MERGE || MODE == MODE_EAGER || MODE == MODE_FOLD || MODE == MODE_AUTO;
    constexpr int CP = LOGGED ? CMAX : 4;        // entry slots in LDS (multiple of 4)
    constexpr int KPASS = LOGGED ? (CMAX + EPP - 1) / EPP : 1;
    constexpr int XR = LOGGED ? (CMAX + RPP - 1) / RPP : 1;  // log value rows per thread
    using TX = typename std::conditional<DELTA, float, TIn>::type;  // value-side log dtype
    using Raw = typename In4<TIn>::raw;
    using RawX = typename In4<TX>::raw;
    static_assert(CMAX % 4 == 0, "entry slots come in groups of four");
    // split replay: the record's scaled key and query, PMV floats per thread
    constexpr int PMV = (2 * DK + NT - 1) / NT;

    __shared__ __attribute__((aligned(16))) float s_mv0[DK];    // khat (delta rules)
    __shared__ __attribute__((aligned(16))) float s_mv1[DK];    // qhat, or rhat (RWKV6)
    __shared__ __attribute__((aligned(16))) float s_scale[DK];  // factor on each base row when writing
    __shared__ __attribute__((aligned(16))) float s_krow[DK];   // current key, per row
    __shared__ __attribute__((aligned(16))) float s_wrow[DK];   // RWKV6: current decay, per row
    __shared__ __attribute__((aligned(16))) float s_kt[LOGGED ? CP * DK : 4];  // [entry][row] decayed keys
    __shared__ __attribute__((aligned(16))) float s_x[LOGGED && CAN_WRITE ? CP * TV : 4];  // [entry][tile col]
    __shared__ float s_coef[2][CP];  // replay coefficients: k side, q/r side
    __shared__ __attribute__((aligned(16))) float s_red[NW][2][TV];
    __shared__ __attribute__((aligned(16))) float s_u[TV];  // current value factor
    __shared__ float s_dot;          // <k,q> (delta rules) or sum r*bonus*k (RWKV6)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int C = p.C;
    int L = LOGGED ? p.L : 0;
    if (LOGGED && p.slot_base != nullptr) {
        // per-slot logs: this slot's own length.  A per-slot decode step is
        // one AUTO launch (append, or fold when this token fills the slot's
        // log) and a per-slot merge or materialise a FOLD launch; APPEND and
        // MERGE, given slot arrays, serve only the slots that stay below C or
        // fill, respectively.  The whole workgroup leaves together, before
        // any barrier.
        const int b = n / p.H;
        if (!p.slot_active[b]) return;
        L = (int)((p.step - (unsigned)p.slot_base[b]) % (unsigned)C);
        if (MODE == MODE_APPEND && L + 1 == C) return;
        if (MODE == MODE_MERGE && L + 1 != C) return;
    }
    // What this workgroup does (uniform across it): compile-time except in
    // AUTO mode, where the token that fills the log also folds it.
    const bool fold = AUTO ? (L + 1 == C) : MODE == MODE_MERGE;
    const bool append = AUTO ? !fold : (MODE == MODE_APPEND || PREP || PREPPED);
    const bool writes = AUTO ? fold : CAN_WRITE;  // writes a dense state
    const bool cur_in_log = fold && DELTA;        // fold the token as entry L
    const int last = L > 0 ? L - 1 : 0;  // newest log entry (clamp target of masked loads)
    const int cg = tid % LPR;            // float4 column group: tile columns 4cg .. 4cg+3
    const int rs = tid / LPR;            // rows rs + RPP*i, i < R
    const int col0 = tile * TV;          // first value column of the tile
    const int c4 = 4 * (tid % KL);       // key-side work: channels c4 .. c4+3
    const int ke = tid / KL;             //   of log entry pass*EPP + ke

    // ---------------- Phase A: issue every load ----------------
    // A1. The token: q (or r), k and the decay of channels c4..c4+3.
    Raw kraw = {}, qraw = {};
    f4 dec4 = {1.f, 1.f, 1.f, 1.f}, bon4 = {0.f, 0.f, 0.f, 0.f};
    float alpha = 1.f, beta = 0.f;
    TIn vraw = {};
    if (TOKEN) {
        if (!PREPPED) {
            kraw = *reinterpret_cast<const Raw *>(static_cast<const TIn *>(p.k) + (size_t)n * DK + c4);
            qraw = *reinterpret_cast<const Raw *>(static_cast<const TIn *>(p.q) + (size_t)n * DK + c4);
            if (GDN)
                alpha = p.decay[n];
            else
                dec4 = *reinterpret_cast<const f4 *>(p.decay + (size_t)n * DK + c4);
        }
        if (DELTA && !PREP) beta = p.beta[n];
        if (OP == OP_RWKV6 && !PREPPED)
            bon4 = *reinterpret_cast<const f4 *>(p.bonus + (size_t)(n % p.H) * DK + c4);
        if (!PREP) vraw = static_cast<const TIn *>(p.v)[(size_t)n * DV + col0 + tid % TV];  // used by tid < TV
    }
    // A2. The log: cumulative log-decay of the newest entry, the key side of
    //     this thread's entries and, in the thread's own row slots (entries
    //     rs + RPP*j), the tile's value side as float4 rows.
    float glast_s = 0.f;
    f4 glast4 = {0.f, 0.f, 0.f, 0.f};
    // A bound above 8 entries (CMAX 16, 32) spreads the key side over KPASS
    // passes and the value side over XR row passes; a pass that holds no
    // logged entry (uniform: it depends only on L) is neither loaded nor
    // computed.  Pass 0 always runs, so the 8-entry kernels are unchanged.
    auto pass_used = [&](int ps) { return ps == 0 || ps * EPP < L; };
    auto row_pass_used = [&](int j) { return j == 0 || RPP * j < L; };
    Raw klog[KPASS];
    float glog_s[KPASS];
    f4 glog4[KPASS];
    RawX xrow[XR];
    if (LOGGED && !PREPPED) {
        const size_t el = (size_t)n * C + last;
        if (GDN)
            glast_s = p.logG[el];
        else
            glast4 = *reinterpret_cast<const f4 *>(p.logG + el * DK + c4);
#pragma unroll
        for (int ps = 0; ps < KPASS; ++ps) {
            if (!pass_used(ps)) continue;
            const size_t e = (size_t)n * C + min(ps * EPP + ke, last);
            klog[ps] = *reinterpret_cast<const Raw *>(static_cast<const TIn *>(p.logK) + e * DK + c4);
            if (GDN)
                glog_s[ps] = p.logG[e];
            else
                glog4[ps] = *reinterpret_cast<const f4 *>(p.logG + e * DK + c4);
        }
    }
    if (LOGGED && !PREP) {
        const TX *xin = static_cast<const TX *>(p.logX) + (size_t)n * C * DV + col0 + 4 * cg;
#pragma unroll
        for (int j = 0; j < XR; ++j)
            if (row_pass_used(j)) xrow[j] = *reinterpret_cast<const RawX *>(xin + (size_t)min(rs + RPP * j, last) * DV);
    }
    // A2'. Split replay: this head's prep record (thread t takes floats t,
    //      t + NT, ... of the scaled key | scaled query, and one coefficient).
    float pre_mv[PMV], pre_coef = 0.f, pre_dot = 0.f;
    if (PREPPED) {
        const float *rec = p.prep + (size_t)n * prep_stride(DK, CMAX);
#pragma unroll
        for (int m = 0; m < PMV; ++m) pre_mv[m] = rec[min(tid + m * NT, 2 * DK - 1)];
        pre_coef = rec[2 * DK + tid % (2 * CP)];
        pre_dot = rec[2 * DK + 2 * CP];
    }

    // A3. The base tile: nearly all of the traffic, issued last so that the
    //     key-side preparation below, which waits only for the small loads
    //     above (loads complete in issue order), overlaps the tile's flight.
    //     Row r of the tile is TV/4 float4 at head offset r*DV/4 + col0/4.
    const size_t tile4 = (size_t)n * (DK * DV / 4) + col0 / 4 + (size_t)rs * (DV / 4) + cg;
    const f4 *src4 = reinterpret_cast<const f4 *>(p.base) + tile4;
    f4 s[R];
    if (!PREP) {
#pragma unroll
        for (int i = 0; i < R; ++i) s[i] = __builtin_nontemporal_load(src4 + (size_t)i * RPP * (DV / 4));
    }

    // ---------------- Phase B: key-side preparation into LDS ----------------
    if constexpr (PREPPED) {
#pragma unroll
        for (int m = 0; m < PMV; ++m) {
            const int idx = tid + m * NT;
            if (idx < DK)
                s_mv0[idx] = pre_mv[m];
            else if (idx < 2 * DK)
                s_mv1[idx - DK] = pre_mv[m];
        }
        if (tid < 2 * CP) (&s_coef[0][0])[tid] = pre_coef;
        if (tid == 0) s_dot = pre_dot;
    } else {
    const f4 k = TOKEN ? In4<TIn>::unpack(kraw) : f4{0.f, 0.f, 0.f, 0.f};
    const f4 q = TOKEN ? In4<TIn>::unpack(qraw) : f4{0.f, 0.f, 0.f, 0.f};
    const f4 dv = GDN ? f4{alpha, alpha, alpha, alpha} : dec4;
    f4 gl, gn, gref, sc;
    if (GDN) {
        const float g0 = L > 0 ? glast_s : 0.f;
        const float g1 = g0 + ((TOKEN && LOGGED) ? log2f(alpha) : 0.f);
        const float gr = (DELTA && TOKEN) ? g1 : g0;
        const float e = MODE == MODE_EAGER ? alpha : exp2f(gr);
        gl = f4{g0, g0, g0, g0};
        gn = f4{g1, g1, g1, g1};
        gref = f4{gr, gr, gr, gr};
        sc = f4{e, e, e, e};
    } else {
        const f4 zero = {0.f, 0.f, 0.f, 0.f};
        gl = L > 0 ? glast4 : zero;
        gn = (TOKEN && LOGGED) ? gl + log2v(dec4) : gl;
        gref = (DELTA && TOKEN) ? gn : gl;
        sc = MODE == MODE_EAGER ? dec4 : exp2v(gref);
    }
    if (ke == 0) {
        // per-row factors of the matrix-vector products and of the state write
        f4 mv0, mv1;
        if (MODE == MODE_EAGER) {
            mv0 = dv * k;
            mv1 = DELTA ? dv * q : q;  // RWKV6 reads the pre-update state
        } else {
            mv0 = sc * k;
            mv1 = sc * q;
        }
        *reinterpret_cast<f4 *>(&s_mv0[c4]) = mv0;
        *reinterpret_cast<f4 *>(&s_mv1[c4]) = mv1;
        *reinterpret_cast<f4 *>(&s_scale[c4]) = sc;
        *reinterpret_cast<f4 *>(&s_krow[c4]) = k;
        *reinterpret_cast<f4 *>(&s_wrow[c4]) = dv;
        if (LOGGED && CAN_WRITE && cur_in_log) *reinterpret_cast<f4 *>(&s_kt[L * DK + c4]) = k;
    }
    // append the token's key side as entry L (one writer per value; tile 0)
    if (append && tile == 0 && ke == 0) {
        const size_t e = (size_t)n * C + L;
        *reinterpret_cast<Raw *>(static_cast<TIn *>(p.logK) + e * DK + c4) = kraw;
        if (!GDN) *reinterpret_cast<f4 *>(p.logG + e * DK + c4) = gn;
    }
    if (append && GDN && tile == 0 && tid == 0) p.logG[(size_t)n * C + L] = gn.x;
    if (TOKEN) {
        // every key-side group holds all DK channels, so each group's sum is complete
        float part = DELTA ? dot4(k, q) : dot4(q * bon4, k);
        part = group_sum_valu<KL>(part);
        if (tid == 0) s_dot = part;
    }
    if (LOGGED) {
        // decayed keys k_i * 2^{g - g_i} and the replay coefficients
        float pk[KPASS], pq[KPASS];
#pragma unroll
        for (int ps = 0; ps < KPASS; ++ps) {
            if (!pass_used(ps)) continue;
            const int i = ps * EPP + ke;
            const bool valid = i < L;
            const f4 kv = In4<TIn>::unpack(klog[ps]);
            f4 kt;
            if (GDN)
                kt = kv * exp2f(gref.x - glog_s[ps]);
            else
                kt = kv * exp2v(gref - glog4[ps]);
            if (!valid) kt = f4{0.f, 0.f, 0.f, 0.f};
            pk[ps] = dot4(kt, k);
            pq[ps] = dot4(kt, q);
            if (CAN_WRITE && writes && valid) *reinterpret_cast<f4 *>(&s_kt[i * DK + c4]) = kt;
        }
        if (TOKEN) {
#pragma unroll
            for (int ps = 0; ps < KPASS; ++ps) {
                if (!pass_used(ps)) continue;
                pk[ps] = group_sum_valu<KL>(pk[ps]);
                pq[ps] = group_sum_valu<KL>(pq[ps]);
            }
            if (c4 == 0) {
#pragma unroll
                for (int ps = 0; ps < KPASS; ++ps) {
                    const int i = ps * EPP + ke;
                    if (pass_used(ps) && i < L) {
                        s_coef[0][i] = pk[ps];
                        s_coef[1][i] = pq[ps];
                    }
                }
            }
        }
        // value side of the log for the fold: this tile's columns of entries 0..L-1
        if (CAN_WRITE && writes) {
#pragma unroll
            for (int j = 0; j < XR; ++j) {
                const int i = rs + RPP * j;
                if (i < L) *reinterpret_cast<f4 *>(&s_x[i * TV + 4 * cg]) = In4<TX>::unpack(xrow[j]);
            }
        }
        // zero the slots between the last folded entry and the next multiple of four
        if (CAN_WRITE && writes) {
            constexpr int W = DK > TV ? DK : TV;
            const int ne = cur_in_log ? L + 1 : L;
            const int pad = ((ne + 3) & ~3) - ne;
            for (int idx = tid; idx < pad * W; idx += NT) {
                const int i = ne + idx / W;
                const int c = idx % W;
                if (c < DK) s_kt[i * DK + c] = 0.f;
                if (c < TV) s_x[i * TV + c] = 0.f;
            }
        }
    }
    }  // phase B computed here (not PREPPED)
    __syncthreads();

    if constexpr (PREP) {
        // split replay, first stage: store the record and leave
        float *rec = p.prep + (size_t)n * prep_stride(DK, CMAX);
        for (int idx = tid; idx < 2 * DK; idx += NT)
            if (DELTA || idx >= DK) rec[idx] = idx < DK ? s_mv0[idx] : s_mv1[idx - DK];
        if (tid < L) {
            rec[2 * DK + tid] = s_coef[0][tid];
            rec[2 * DK + CP + tid] = s_coef[1][tid];
        }
        if (tid == 0) rec[2 * DK + 2 * CP] = s_dot;
        return;
    }

    if (TOKEN) {
        // ---------------- Phase C: matrix-vector products ----------------
        f4 y = {0.f, 0.f, 0.f, 0.f}, z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int row = rs + RPP * i;
            if (DELTA) y += s[i] * s_mv0[row];
            z += s[i] * s_mv1[row];
        }
        // the log replay joins the same reduction: entry i = rs + RPP*j adds
        // coef_i * x_i to the partial sums of the thread holding row slot rs
        if (LOGGED) {
#pragma unroll
            for (int j = 0; j < XR; ++j) {
                const int i = rs + RPP * j;
                if (i < L) {
                    const f4 x = In4<TX>::unpack(xrow[j]);
                    if (DELTA) y += s_coef[0][i] * x;
                    z += s_coef[1][i] * x;
                }
            }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (DELTA) y[c] = column_sum_valu<LPR>(y[c]);
            z[c] = column_sum_valu<LPR>(z[c]);
        }
        if (lane < LPR) {
            if (DELTA) *reinterpret_cast<f4 *>(&s_red[wave][0][4 * cg]) = y;
            *reinterpret_cast<f4 *>(&s_red[wave][1][4 * cg]) = z;
        }
        __syncthreads();

        // ---------------- Phase D: column stage, one thread per tile column ----------------
        if (tid < TV) {
            const int jt = tid;       // column within the tile
            const int j = col0 + jt;  // column within the head
            float yj = 0.f, zj = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                if (DELTA) yj += s_red[w][0][jt];
                zj += s_red[w][1][jt];
            }
            const float vj = to_f32(vraw);
            float xnew, o;
            if (DELTA) {
                xnew = beta * (vj - yj);
                o = zj + s_dot * xnew;
            } else {
                xnew = vj;
                o = zj + s_dot * vj;
            }
            p.out[(size_t)n * DV + j] = o;
            if (append) {
                const size_t e = (size_t)n * C + L;
                if (DELTA)
                    static_cast<float *>(p.logX)[e * DV + j] = xnew;
                else
                    static_cast<TIn *>(p.logX)[e * DV + j] = vraw;
            }
            if (LOGGED && CAN_WRITE && cur_in_log)
                s_x[L * TV + jt] = xnew;
            else
                s_u[jt] = xnew;
        }
        if (CAN_WRITE && writes) __syncthreads();
    }

    if (CAN_WRITE && writes) {
        // ---------------- Phase E: write the state ----------------
        // row scale, the rank-(entries) update from LDS, then the current
        // token for RWKV6 and the eager form.
        const int ne = cur_in_log ? L + 1 : L;
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
                    const int row = rs + RPP * i;
                    acc[i] += s_kt[(e + 0) * DK + row] * x0 + s_kt[(e + 1) * DK + row] * x1 +
                              s_kt[(e + 2) * DK + row] * x2 + s_kt[(e + 3) * DK + row] * x3;
                }
            }
        }
        if (TOKEN && !cur_in_log) {
            const f4 u = *reinterpret_cast<const f4 *>(&s_u[4 * cg]);
#pragma unroll
            for (int i = 0; i < R; ++i) {
                const int row = rs + RPP * i;
                if (fold)  // RWKV6: decay the logical state, then add k v^T
                    acc[i] = acc[i] * s_wrow[row] + s_krow[row] * u;
                else
                    acc[i] += s_krow[row] * u;
            }
        }
        f4 *dst4 = reinterpret_cast<f4 *>(p.dst) + tile4;
#pragma unroll
        for (int i = 0; i < R; ++i) __builtin_nontemporal_store(acc[i], dst4 + (size_t)i * RPP * (DV / 4));
    }
}

// One workgroup per (head, tile), mapped as block_to_tile says.
template <int OP, typename TIn, int DK, int DV, int TV, int NT, int MODE, int CMAX>
__global__ __launch_bounds__(NT) DLK_OCCUPANCY void step_kernel(const StepParams p) {
    int n, tile;
    block_to_tile<StepOrder<DK, DV>::XCD>(blockIdx.x, p.N, MODE == MODE_PREP ? 1 : DV / TV, n, tile);
    step_body<OP, TIn, DK, DV, TV, NT, MODE, CMAX>(p, n, tile);
}

// Whole heads, except the last `tail` heads of the launch, which run as two
// half-width tiles each on the same number of threads.  Workgroups start in
// dispatch order, so the last ones to start set the launch's end; with half
// a head's bytes each they end about half a workgroup lifetime sooner.
template <int OP, typename TIn, int DK, int DV, int NT, int MODE, int CMAX>
__global__ __launch_bounds__(NT) DLK_OCCUPANCY void step_kernel_tail(const StepParams p, const int tail) {
    const int nf = p.N - tail;
    const int b = blockIdx.x;
    int n, tile;
    if (b < nf) {
        block_to_tile<true>(b, nf, 1, n, tile);
        step_body<OP, TIn, DK, DV, DV, NT, MODE, CMAX>(p, n, 0);
    } else {
        block_to_tile<true>(b - nf, tail, 2, n, tile);
        step_body<OP, TIn, DK, DV, DV / 2, NT, MODE, CMAX>(p, nf + n, tile);
    }
}

}  // namespace dlk
