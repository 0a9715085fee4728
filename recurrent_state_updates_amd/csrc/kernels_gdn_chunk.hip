// Multi-token kernel instantiations for the GDN operator (see chunk_kernel.h).
#include "chunk_kernel.h"

namespace dlk {

hipError_t launch_gdn_chunk(int in_bf16, int D, int cmax, const ChunkParams &p, hipStream_t s) {
    return launch_chunk_op<OP_GDN>(in_bf16, D, cmax, p, s);
}

}  // namespace dlk
