// step_launch.h -- host-side dispatch of the single-token kernel family:
// (operator, input dtype, key width, value width, mode, log bound) -> one
// instantiation of step_kernel and its grid.
#pragma once

#include "step_kernel.h"

namespace dlk {

// At 128 x 128 the decode modes of the kernels built for 8-entry logs run
// the launch's last TAIL_HEADS_128 heads as two half-width tiles each
// (step_kernel_tail) when the launch has at least four times as many heads
// (two or more rounds of workgroups on the chip).  Measured on MI355X at
// B=128, H=32, C=8 (two alternating runs): GDN 51.35-51.45 against
// 52.03-52.12 us/token back to back, KDA 54.16-54.19 against 54.90-55.01,
// and the same with the cache refilled before every launch; 256 tail heads
// did as well, 1024 half as well.  The kernels built for 16 and 32 entries
// keep whole heads: with both tile forms in one kernel their folds need
// 169-193 VGPRs, two waves per SIMD instead of four (a fold at C=32 took
// 129 instead of 109 us).  The 64 x 64 heads keep whole heads too: there
// the half tiles slowed RWKV6's folds.
constexpr int TAIL_HEADS_128 = 512;

template <int OP, typename TIn, int DK, int DV, int MODE, int CMAX>
hipError_t launch_one(const StepParams &p, hipStream_t s) {
    constexpr int TV = Shape<DK, DV, MODE>::TV, NT = Shape<DK, DV, MODE>::NT;
    if constexpr (DK == 128 && DV == 128 && TV == DV && CMAX == 8 &&
                  (MODE == MODE_APPEND || MODE == MODE_MERGE || MODE == MODE_AUTO)) {
        if (p.N >= 4 * TAIL_HEADS_128) {
            const unsigned blocks = (unsigned)(p.N + TAIL_HEADS_128);
            hipLaunchKernelGGL((step_kernel_tail<OP, TIn, DK, DV, NT, MODE, CMAX>), dim3(blocks), dim3(NT), 0, s, p,
                               TAIL_HEADS_128);
            return hipGetLastError();
        }
    }
    const unsigned blocks = (unsigned)p.N * (MODE == MODE_PREP ? 1 : DV / TV);
    hipLaunchKernelGGL((step_kernel<OP, TIn, DK, DV, TV, NT, MODE, CMAX>), dim3(blocks), dim3(NT), 0, s, p);
    return hipGetLastError();
}

// The instantiation whose log bound covers cmax: 8, 16 or 32 entries (a
// larger bound holds more key-side registers, so each capacity gets the
// smallest that fits).
template <int OP, typename TIn, int DK, int DV, int MODE>
hipError_t launch_bounded(int cmax, const StepParams &p, hipStream_t s) {
    if (cmax <= 8) return launch_one<OP, TIn, DK, DV, MODE, 8>(p, s);
    if (cmax <= 16) return launch_one<OP, TIn, DK, DV, MODE, 16>(p, s);
    return launch_one<OP, TIn, DK, DV, MODE, 32>(p, s);
}

template <int OP, typename TIn, int DK, int DV>
hipError_t launch_mode(int mode, int cmax, const StepParams &p, hipStream_t s) {
    switch (mode) {
        case MODE_APPEND: return launch_bounded<OP, TIn, DK, DV, MODE_APPEND>(cmax, p, s);
        case MODE_MERGE: return launch_bounded<OP, TIn, DK, DV, MODE_MERGE>(cmax, p, s);
        case MODE_FOLD: return launch_bounded<OP, TIn, DK, DV, MODE_FOLD>(cmax, p, s);
        case MODE_AUTO: return launch_bounded<OP, TIn, DK, DV, MODE_AUTO>(cmax, p, s);
        case MODE_PREP: return launch_bounded<OP, TIn, DK, DV, MODE_PREP>(cmax, p, s);
        case MODE_PREPPED: return launch_bounded<OP, TIn, DK, DV, MODE_PREPPED>(cmax, p, s);
        case MODE_EAGER:
            return launch_one<OP, TIn, DK, DV, MODE_EAGER, 4>(p, s);
        default:
            return hipErrorInvalidValue;
    }
}

template <int OP, typename TIn, int DK>
hipError_t launch_value_width(int DV, int mode, int cmax, const StepParams &p, hipStream_t s) {
    switch (DV) {
        case 32: return launch_mode<OP, TIn, DK, 32>(mode, cmax, p, s);
        case 64: return launch_mode<OP, TIn, DK, 64>(mode, cmax, p, s);
        case 128: return launch_mode<OP, TIn, DK, 128>(mode, cmax, p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dlk
