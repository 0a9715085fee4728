// Single-token kernel instantiations for one operator and one key width
// (see step_kernel.h).  The build compiles this file once per pair, with
// -DDLK_OP=0|1|2 (GDN, KDA, RWKV6) and -DDLK_DK=32|64|128, so that the
// translation units compile in parallel.
#include "step_launch.h"

namespace dlk {

template <int OP, int DK>
hipError_t launch_step(int in_bf16, int DV, int mode, int cmax, const StepParams &p, hipStream_t s) {
    return in_bf16 ? launch_value_width<OP, bf16_bits, DK>(DV, mode, cmax, p, s)
                   : launch_value_width<OP, float, DK>(DV, mode, cmax, p, s);
}

template hipError_t launch_step<DLK_OP, DLK_DK>(int, int, int, int, const StepParams &, hipStream_t);

}  // namespace dlk
