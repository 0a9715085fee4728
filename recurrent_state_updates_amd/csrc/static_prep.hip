// static_prep.hip -- the scratch of the allocation-free decode step
// (dl_decode_step_noalloc): the split replay's per-head prep records in a
// file-scope device array instead of a caller buffer.  Each GPU the library
// runs on holds its own copy of the array, at its own address, from the
// moment the library's code is loaded on it until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/deltalog.h"
#include "launch.h"

namespace {

// Host code must not pass `scratch` itself to a kernel: on the host the name
// is a stand-in, not a device address.  The device address of each GPU's
// copy comes from hipGetSymbolAddress, with that GPU current.
static __device__ __align__(256) unsigned char scratch[DL_NOALLOC_PREP_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices];

}  // namespace

namespace dlk {

hipError_t static_prep_scratch(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    return hipSuccess;
}

}  // namespace dlk
