// stub_launch.h -- what the stub launchers of the host-only build record.
#pragma once

#include <vector>

#include "../../recurrent_state_updates_amd/csrc/launch.h"

namespace dlk {

enum { KIND_STEP = 0, KIND_CHUNK = 1, KIND_SLOT_SET = 2 };

struct Launch {
    int kind;
    // KIND_STEP / KIND_CHUNK
    int op, dk, dv, mode, cmax, L, C, N, K, segmented;
    bool slots, prep;
    unsigned step;
    // KIND_SLOT_SET
    int B, slot, set_base, base_value, set_active, active_value, only_active;
};

extern std::vector<Launch> g_launches;

}  // namespace dlk
