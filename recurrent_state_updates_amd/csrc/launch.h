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

// Floats in one head's prep record for key width DK and log bound cmax:
// [0, DK) scaled key, [DK, 2DK) scaled query (or receptance), then cmax
// key-side and cmax query-side replay coefficients, then the token's scalar
// term.
constexpr int prep_stride(int DK, int cmax) { return 2 * DK + 2 * cmax + 4; }

struct StepParams {
    float *base;         // [N][DK][DV] fp32 base (or dense state for EAGER)
    float *dst;          // state written by MERGE / EAGER / FOLD
    const void *q;       // [N][DK] input dtype: q (GDN, KDA) or r (RWKV6)
    const void *k;       // [N][DK] input dtype
    const void *v;       // [N][DV] input dtype
    const float *beta;   // [N]
    const float *decay;  // [N] (GDN) or [N][DK]
    const float *bonus;  // [H][DK] (RWKV6)
    float *out;          // [N][DV] fp32
    void *logX;          // [N][C][DV]: fp32 (GDN, KDA) or input dtype (RWKV6)
    void *logK;          // [N][C][DK] input dtype
    float *logG;         // [N][C] (GDN) or [N][C][DK] fp32, base-2 cumulative log-decay
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
    float *prep;                       // [N][prep_stride(DK, cmax)] split-replay records
};

// Launch one mode of the single-token kernel for operator OP and key width
// DK (32, 64 or 128).  in_bf16 selects the input dtype, DV the value width
// (32, 64 or 128), cmax the compile-time bound on log entries (8, 16 or 32).
// Defined in step_launch.h; each (OP, DK) is instantiated in a translation
// unit of its own (kernels_step.hip compiled with -DDLK_OP, -DDLK_DK).
template <int OP, int DK>
hipError_t launch_step(int in_bf16, int DV, int mode, int cmax, const StepParams &p, hipStream_t s);

// Several consecutive tokens of every head in one launch (lockstep or per-slot logs).
constexpr int KMAX_TOKENS = 8;
struct ChunkParams {
    float *base;                        // [N][DK][DV] fp32, rewritten in place when fold
    const void *q[KMAX_TOKENS];         // token t: [N][DK] input dtype (v: [N][DV])
    const void *k[KMAX_TOKENS];
    const void *v[KMAX_TOKENS];
    const float *beta[KMAX_TOKENS];     // [N] (GDN, KDA)
    const float *decay[KMAX_TOKENS];    // [N] (GDN) or [N][DK]
    float *out[KMAX_TOKENS];            // [N][DV] fp32
    const float *bonus;                 // [H][DK] (RWKV6)
    void *logX;
    void *logK;
    float *logG;
    int L;     // log entries before the chunk, L < C
    int C;     // capacity
    int H;
    int N;
    int K;     // tokens in the chunk, 1 <= K <= KMAX_TOKENS
    // The kernel folds the log's first C entries into the base when L + K >= C
    // and starts the new log with the tokens past the fold.  segmented == 0
    // requires K <= C (at most one fold per call); segmented != 0 (K > C, so
    // C < KMAX_TOKENS) folds each time the log fills.  On per-slot handles
    // (slot_base != NULL) each slot's log length is (step - slot_base[b]) mod C,
    // and L is ignored.
    int segmented;
    const int *slot_base;
    const unsigned char *slot_active;
    unsigned step;
};

// The multi-token kernel for operator OP and key width DK; defined in
// chunk_kernel.h, instantiated per (OP, DK) in kernels_chunk.hip.
template <int OP, int DK>
hipError_t launch_chunk(int in_bf16, int DV, int cmax, const ChunkParams &p, hipStream_t s);

// The device address of this GPU's copy of the allocation-free decode
// step's scratch (DL_NOALLOC_PREP_BYTES bytes; static_prep.hip), looked up
// once per device with that device current.
hipError_t static_prep_scratch(void **ptr);

// Set slot_base / slot_active entries: slot < 0 means every slot (with
// only_active, every active slot); set_base / set_active select the fields.
hipError_t launch_slot_set(int *slot_base, unsigned char *slot_active, int B, int slot, int set_base,
                           int base_value, int set_active, int active_value, int only_active,
                           hipStream_t s);

}  // namespace dlk
