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
enum { MODE_APPEND = 0, MODE_MERGE = 1, MODE_EAGER = 2, MODE_FOLD = 3 };

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
};

// Launch one mode for one operator.  in_bf16 selects the input dtype, D the
// head width (dk == dv), cmax the compile-time bound on log entries (8 or 32).
hipError_t launch_gdn(int in_bf16, int D, int mode, int cmax, const StepParams &p, hipStream_t s);
hipError_t launch_kda(int in_bf16, int D, int mode, int cmax, const StepParams &p, hipStream_t s);
hipError_t launch_rwkv6(int in_bf16, int D, int mode, int cmax, const StepParams &p, hipStream_t s);

}  // namespace dlk
