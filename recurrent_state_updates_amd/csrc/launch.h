// launch.h -- internal interface between the C-ABI host code and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace dlk {

enum { OP_GDN = 0, OP_KDA = 1, OP_RWKV6 = 2 };

// What one launch does to each head.
//   APPEND  decode a token against base + log, append its factors as entry L
//   MERGE   decode a token (L = C-1 entries logged) and fold all C into the base
//   EAGER   decode a token directly on a dense state (no log), rewrite it
//   FOLD    write base + log (L entries) to dst; no token
//   AUTO    per slot: APPEND, or MERGE when the token fills the slot's log
//   PREP    split replay, first stage: once per head (one workgroup each),
//           the token's key-side preparation -- scaled key and query, the
//           replay coefficients of the L logged entries and <k,q> -- written
//           to a prep record, and the key side of entry L appended
//   PREPPED split replay, second stage: APPEND with the key side read from
//           the prep record instead of computed
enum { MODE_APPEND = 0, MODE_MERGE = 1, MODE_EAGER = 2, MODE_FOLD = 3, MODE_AUTO = 4, MODE_PREP = 5,
       MODE_PREPPED = 6 };

// Floats in one head's prep record for head width D and log bound cmax:
// [0, D) scaled key, [D, 2D) scaled query (or receptance), then cmax key-side
// and cmax query-side replay coefficients, then the token's scalar term.
constexpr int prep_stride(int D, int cmax) { return 2 * D + 2 * cmax + 4; }

struct StepParams {
    float *base;         // [N][D][D] fp32 base (or dense state for EAGER)
    float *dst;          // state written by MERGE / EAGER / FOLD
    const void *q;       // [N][D] input dtype: q (GDN, KDA) or r (RWKV6)
    const void *k;       // [N][D] input dtype
    const void *v;       // [N][D] input dtype
    const float *beta;   // [N]
    const float *decay;  // [N] (GDN) or [N][D]
    const float *bonus;  // [H][D] (RWKV6)
    float *out;          // [N][D] fp32
    void *logX;          // [N][C][D]: fp32 (GDN, KDA) or input dtype (RWKV6)
    void *logK;          // [N][C][D] input dtype
    float *logG;         // [N][C] (GDN) or [N][C][D] fp32, base-2 cumulative log-decay
    int L;               // log entries present before the launch
    int C;               // log capacity (entry stride of the log arrays)
    int H;               // heads per slot (bonus row = n % H)
    int N;               // heads = grid size
    // Per-slot logs (continuous batching); slot_base == nullptr selects the
    // lockstep log of length L.  Slot b's log length is
    // (step - slot_base[b]) mod C; inactive slots are skipped.
    const int *slot_base;              // [B] decode-step index of the slot's last empty log
    const unsigned char *slot_active;  // [B] 1 = decode this slot
    unsigned step;                     // decode steps issued so far
    float *prep;                       // [N][prep_stride(D, cmax)] split-replay records
};

// Launch one mode for one operator.  in_bf16 selects the input dtype, D the
// head width (dk == dv), cmax the compile-time bound on log entries (8, 16 or 32).
hipError_t launch_gdn(int in_bf16, int D, int mode, int cmax, const StepParams &p, hipStream_t s);
hipError_t launch_kda(int in_bf16, int D, int mode, int cmax, const StepParams &p, hipStream_t s);
hipError_t launch_rwkv6(int in_bf16, int D, int mode, int cmax, const StepParams &p, hipStream_t s);

// Several consecutive tokens of every head in one launch (lockstep or per-slot logs).
constexpr int KMAX_TOKENS = 8;
struct ChunkParams {
    float *base;                        // [N][D][D] fp32, rewritten in place when fold
    const void *q[KMAX_TOKENS];         // token t: [N][D] input dtype
    const void *k[KMAX_TOKENS];
    const void *v[KMAX_TOKENS];
    const float *beta[KMAX_TOKENS];     // [N] (GDN, KDA)
    const float *decay[KMAX_TOKENS];    // [N] (GDN) or [N][D]
    float *out[KMAX_TOKENS];            // [N][D] fp32
    const float *bonus;                 // [H][D] (RWKV6)
    void *logX;
    void *logK;
    float *logG;
    int L;     // log entries before the chunk
    int C;     // capacity; L + K <= C
    int H;
    int N;
    int K;     // tokens in the chunk, 1 <= K <= KMAX_TOKENS
    int fold;  // 1: L + K == C, fold every entry into the base
    // segmented != 0: the K tokens may pass the log's end; the kernel folds
    // when the log fills and starts an empty log for the rest (fold is then
    // ignored).  Per-slot handles (slot_base != NULL) are always segmented:
    // each slot's log length is (step - slot_base[b]) mod C, and L is ignored.
    int segmented;
    const int *slot_base;
    const unsigned char *slot_active;
    unsigned step;
};

hipError_t launch_gdn_chunk(int in_bf16, int D, int cmax, const ChunkParams &p, hipStream_t s);
hipError_t launch_kda_chunk(int in_bf16, int D, int cmax, const ChunkParams &p, hipStream_t s);
hipError_t launch_rwkv6_chunk(int in_bf16, int D, int cmax, const ChunkParams &p, hipStream_t s);

// Set slot_base / slot_active entries: slot < 0 means every slot (with
// only_active, every active slot); set_base / set_active select the fields.
hipError_t launch_slot_set(int *slot_base, unsigned char *slot_active, int B, int slot, int set_base,
                           int base_value, int set_active, int active_value, int only_active,
                           hipStream_t s);

}  // namespace dlk
