// step_launch.h -- host-side dispatch of the single-token kernel family:
// (operator, input dtype, key width, value width, mode, log bound) -> one
// instantiation of step_kernel and its grid.
#pragma once

#include "step_kernel.h"

namespace dlk {

template <int OP, typename TIn, int DK, int DV, int MODE, int CMAX>
hipError_t launch_one(const StepParams &p, hipStream_t s) {
    constexpr int TV = Shape<DK, DV, MODE>::TV, NT = Shape<DK, DV, MODE>::NT;
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
