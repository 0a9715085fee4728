// stub_launch.cpp -- kernel launchers for a host-only build of the library:
// each records what the host code asked for and returns success without
// touching a device, so that the validation, the log-length bookkeeping and
// the choice of launch mode can run (under the address and undefined-
// behaviour sanitizers) on a machine without a GPU.  Test infrastructure.
#include "stub_launch.h"

#include <stdint.h>

namespace dlk {

std::vector<Launch> g_launches;

template <int OP, int DK>
hipError_t launch_step(int, int DV, int mode, int cmax, const StepParams &p, hipStream_t) {
    Launch l = {};
    l.kind = KIND_STEP;
    l.op = OP, l.dk = DK, l.dv = DV, l.mode = mode, l.cmax = cmax, l.L = p.L, l.C = p.C, l.N = p.N, l.K = 1;
    l.slots = p.slot_base != nullptr, l.prep = p.prep != nullptr, l.step = p.step;
    g_launches.push_back(l);
    return hipSuccess;
}

template <int OP, int DK>
hipError_t launch_chunk(int, int DV, int cmax, const ChunkParams &p, hipStream_t) {
    Launch l = {};
    l.kind = KIND_CHUNK;
    l.op = OP, l.dk = DK, l.dv = DV, l.mode = -1, l.cmax = cmax, l.L = p.L, l.C = p.C, l.N = p.N, l.K = p.K;
    l.segmented = p.segmented, l.slots = p.slot_base != nullptr, l.step = p.step;
    g_launches.push_back(l);
    return hipSuccess;
}

hipError_t launch_slot_set(int *, unsigned char *, int B, int slot, int set_base, int base_value, int set_active,
                           int active_value, int only_active, hipStream_t) {
    Launch l = {};
    l.kind = KIND_SLOT_SET;
    l.B = B, l.slot = slot, l.set_base = set_base, l.base_value = base_value, l.set_active = set_active;
    l.active_value = active_value, l.only_active = only_active;
    g_launches.push_back(l);
    return hipSuccess;
}

// A fake address standing for the static scratch of dl_decode_step_noalloc.
hipError_t static_prep_scratch(void **ptr) {
    *ptr = reinterpret_cast<void *>(static_cast<uintptr_t>(0x7e0000000000ull));
    return hipSuccess;
}

#define DLK_STUBS(OP)                                                                                   \
    template hipError_t launch_step<OP, 32>(int, int, int, int, const StepParams &, hipStream_t);      \
    template hipError_t launch_step<OP, 64>(int, int, int, int, const StepParams &, hipStream_t);      \
    template hipError_t launch_step<OP, 128>(int, int, int, int, const StepParams &, hipStream_t);     \
    template hipError_t launch_chunk<OP, 32>(int, int, int, const ChunkParams &, hipStream_t);         \
    template hipError_t launch_chunk<OP, 64>(int, int, int, const ChunkParams &, hipStream_t);         \
    template hipError_t launch_chunk<OP, 128>(int, int, int, const ChunkParams &, hipStream_t);
DLK_STUBS(0)
DLK_STUBS(1)
DLK_STUBS(2)

}  // namespace dlk
