// Kernel instantiations for the RWKV6 operator (see step_kernel.h).
#include "step_launch.h"

namespace dlk {

hipError_t launch_rwkv6(int in_bf16, int D, int mode, int cmax, const StepParams &p, hipStream_t s) {
    return launch_op<OP_RWKV6>(in_bf16, D, mode, cmax, p, s);
}

}  // namespace dlk
