// slots.hip -- the one-thread-per-slot kernel that activates, deactivates and
// resets per-slot logs (continuous batching).  A plain kernel rather than a
// memset so that a captured graph replays it faithfully.
#include "launch.h"

namespace dlk {

__global__ void slot_set_kernel(int *slot_base, unsigned char *slot_active, int B, int slot, int set_base,
                                int base_value, int set_active, int active_value, int only_active) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B || (slot >= 0 && b != slot)) return;
    if (only_active && !slot_active[b]) return;
    if (set_base) slot_base[b] = base_value;
    if (set_active) slot_active[b] = (unsigned char)active_value;
}

hipError_t launch_slot_set(int *slot_base, unsigned char *slot_active, int B, int slot, int set_base,
                           int base_value, int set_active, int active_value, int only_active,
                           hipStream_t s) {
    const int threads = 256;
    const int blocks = (B + threads - 1) / threads;
    hipLaunchKernelGGL(slot_set_kernel, dim3(blocks), dim3(threads), 0, s, slot_base, slot_active, B, slot,
                       set_base, base_value, set_active, active_value, only_active);
    return hipGetLastError();
}

}  // namespace dlk
