// step_launch.h -- host-side dispatch of the single-token kernel family:
// (operator, input dtype, head width, mode, log bound) -> one instantiation
// of step_kernel and its grid.
#pragma once

#include "step_kernel.h"

namespace dlk {

template <int OP, typename TIn, int D, int MODE, int CMAX>
hipError_t launch_one(const StepParams &p, hipStream_t s) {
    constexpr int TV = Shape<D, MODE>::TV, NT = Shape<D, MODE>::NT;
    const unsigned blocks = (unsigned)p.N * (MODE == MODE_PREP ? 1 : D / TV);
    hipLaunchKernelGGL((step_kernel<OP, TIn, D, TV, NT, MODE, CMAX>), dim3(blocks), dim3(NT), 0, s, p);
    return hipGetLastError();
}

// The instantiation whose log bound covers cmax: 8, 16 or 32 entries (a
// larger bound holds more key-side registers, so each capacity gets the
// smallest that fits).
template <int OP, typename TIn, int D, int MODE>
hipError_t launch_bounded(int cmax, const StepParams &p, hipStream_t s) {
    if (cmax <= 8) return launch_one<OP, TIn, D, MODE, 8>(p, s);
    if (cmax <= 16) return launch_one<OP, TIn, D, MODE, 16>(p, s);
    return launch_one<OP, TIn, D, MODE, 32>(p, s);
}

template <int OP, typename TIn, int D>
hipError_t launch_mode(int mode, int cmax, const StepParams &p, hipStream_t s) {
    switch (mode) {
        case MODE_APPEND: return launch_bounded<OP, TIn, D, MODE_APPEND>(cmax, p, s);
        case MODE_MERGE: return launch_bounded<OP, TIn, D, MODE_MERGE>(cmax, p, s);
        case MODE_FOLD: return launch_bounded<OP, TIn, D, MODE_FOLD>(cmax, p, s);
        case MODE_AUTO: return launch_bounded<OP, TIn, D, MODE_AUTO>(cmax, p, s);
        case MODE_PREP: return launch_bounded<OP, TIn, D, MODE_PREP>(cmax, p, s);
        case MODE_PREPPED: return launch_bounded<OP, TIn, D, MODE_PREPPED>(cmax, p, s);
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
