// Multi-token kernel instantiations for one operator and one key width (see
// chunk_kernel.h).  The build compiles this file once per pair, with
// -DDLK_OP=0|1|2 (GDN, KDA, RWKV6) and -DDLK_DK=32|64|128.
#include "chunk_kernel.h"

namespace dlk {

template hipError_t launch_chunk<DLK_OP, DLK_DK>(int, int, int, const ChunkParams &, hipStream_t);

}  // namespace dlk
