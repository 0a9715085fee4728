// probe.hip -- what MI355X streams at the access pattern of the decode
// kernels: the same workgroup per head, thread geometry, block order and
// 16-byte nontemporal loads (and stores) as the append and the
// decode-and-fold, with none of their other work.  These bound the path from
// above: an append cannot beat a read of its heads, a fold cannot beat an
// in-place copy of them.  A write of every head (no read) shows what the
// write side alone streams, beside the copy that mixes the two.
#include "../../include/deltalog_probe.h"

#include <hip/hip_runtime.h>

#include <string>

#include "step_launch.h"

namespace dlk {

// KIND = DL_PROBE_READ: read every head once and keep one conditional store,
// which the compiler cannot drop without the sum (a sum of finite state
// values equal to NaN never happens).  DL_PROBE_COPY: read and write every
// head back in place, multiplied by `one` (1.0f at run time: the values do
// not change, but the compiler cannot drop a store it does not know to be
// redundant).  DL_PROBE_WRITE: write `one` to every element, no read.
template <int DK, int DV, int TV, int NT, int KIND>
__device__ __forceinline__ void probe_body(float *state, float *sink, int n, int tile, float one) {
    using G = Geom<DK, DV, TV, NT>;
    const int tid = threadIdx.x;
    const int cg = tid % G::LPR, rs = tid / G::LPR;
    f4 *p4 = reinterpret_cast<f4 *>(state) + (size_t)n * (DK * DV / 4) + tile * (TV / 4) + (size_t)rs * (DV / 4) + cg;
    if constexpr (KIND == DL_PROBE_WRITE) {
        const f4 c = {one, one, one, one};
#pragma unroll
        for (int i = 0; i < G::R; ++i) __builtin_nontemporal_store(c, p4 + (size_t)i * G::RPP * (DV / 4));
        return;
    }
    f4 s[G::R];
#pragma unroll
    for (int i = 0; i < G::R; ++i) s[i] = __builtin_nontemporal_load(p4 + (size_t)i * G::RPP * (DV / 4));
    if constexpr (KIND == DL_PROBE_COPY) {
#pragma unroll
        for (int i = 0; i < G::R; ++i) __builtin_nontemporal_store(s[i] * one, p4 + (size_t)i * G::RPP * (DV / 4));
    } else {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < G::R; ++i) acc += (s[i].x + s[i].y) + (s[i].z + s[i].w);
        if (acc != acc) sink[0] = acc;
    }
}

// One workgroup per head in the decode kernels' block order; at 128 x 128,
// where the decode kernels of 8-entry logs split the launch's last heads
// into half-width tiles (TAIL_HEADS_128, step_launch.h), the probe does the
// same (it follows those kernels, which serve every capacity up to 8).
template <int DK, int DV, int NT, int KIND>
__global__ __launch_bounds__(NT) void probe_kernel(float *state, float *sink, int N, int tail, float one) {
    const int nf = N - tail;
    const int b = blockIdx.x;
    int n, tile;
    if (b < nf) {
        block_to_tile<StepOrder<DK, DV>::XCD>(b, nf, 1, n, tile);
        probe_body<DK, DV, DV, NT, KIND>(state, sink, n, 0, one);
    } else if constexpr (DV % 8 == 0) {
        block_to_tile<true>(b - nf, tail, 2, n, tile);
        probe_body<DK, DV, DV / 2, NT, KIND>(state, sink, nf + n, tile, one);
    }
}

template <int DK, int DV, int KIND>
void launch_probe_kind(float *state, float *sink, int N, hipStream_t s) {
    constexpr int NT = Shape<DK, DV, MODE_APPEND>::NT;
    const int tail = (DK == 128 && DV == 128 && N >= 4 * TAIL_HEADS_128) ? TAIL_HEADS_128 : 0;
    hipLaunchKernelGGL((probe_kernel<DK, DV, NT, KIND>), dim3(N + tail), dim3(NT), 0, s, state, sink, N, tail, 1.0f);
}

template <int DK, int DV>
hipError_t launch_probe(int kind, float *state, float *sink, int N, hipStream_t s) {
    if (kind == DL_PROBE_COPY)
        launch_probe_kind<DK, DV, DL_PROBE_COPY>(state, sink, N, s);
    else if (kind == DL_PROBE_WRITE)
        launch_probe_kind<DK, DV, DL_PROBE_WRITE>(state, sink, N, s);
    else
        launch_probe_kind<DK, DV, DL_PROBE_READ>(state, sink, N, s);
    return hipGetLastError();
}

template <int DK>
hipError_t probe_value_width(int dv, int kind, float *state, float *sink, int N, hipStream_t s) {
    switch (dv) {
        case 32: return launch_probe<DK, 32>(kind, state, sink, N, s);
        case 64: return launch_probe<DK, 64>(kind, state, sink, N, s);
        case 128: return launch_probe<DK, 128>(kind, state, sink, N, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dlk

namespace {
thread_local std::string g_probe_error;
}

extern "C" {

int dl_probe_stream(int mode, float *state, int B, int H, int dk, int dv, float *sink, void *stream) {
    auto built = [](int w) { return w == 32 || w == 64 || w == 128; };
    if (mode != DL_PROBE_READ && mode != DL_PROBE_COPY && mode != DL_PROBE_WRITE) {
        g_probe_error = "mode must be DL_PROBE_READ, DL_PROBE_COPY or DL_PROBE_WRITE";
        return -1;
    }
    if (!state || !sink || (reinterpret_cast<uintptr_t>(state) & 15u) || (reinterpret_cast<uintptr_t>(sink) & 3u)) {
        g_probe_error = "state (16-byte aligned) and sink (4-byte aligned) must be non-NULL";
        return -1;
    }
    if (B <= 0 || H <= 0 || (size_t)B * (size_t)H > (size_t)(1 << 23)) {
        g_probe_error = "B and H must be positive with B * H <= 2^23";
        return -2;
    }
    if (!built(dk) || !built(dv)) {
        g_probe_error = "dk and dv must each be 32, 64 or 128";
        return -3;
    }
    const int N = B * H;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    switch (dk) {
        case 32: e = dlk::probe_value_width<32>(dv, mode, state, sink, N, s); break;
        case 64: e = dlk::probe_value_width<64>(dv, mode, state, sink, N, s); break;
        default: e = dlk::probe_value_width<128>(dv, mode, state, sink, N, s); break;
    }
    if (e != hipSuccess) {
        g_probe_error = std::string("kernel launch failed: ") + hipGetErrorString(e);
        return -4;
    }
    g_probe_error.clear();
    return 0;
}

const char *dl_probe_last_error(void) { return g_probe_error.c_str(); }

}  // extern "C"
