// Multi-token kernel instantiations for the KDA operator (see chunk_kernel.h).
#include "chunk_kernel.h"

namespace dlk {

hipError_t launch_kda_chunk(int in_bf16, int D, int cmax, const ChunkParams &p, hipStream_t s) {
    return launch_chunk_op<OP_KDA>(in_bf16, D, cmax, p, s);
}

}  // namespace dlk
