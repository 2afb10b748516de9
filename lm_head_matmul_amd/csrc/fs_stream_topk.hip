// fs_stream_topk.hip -- streaming kernels with the fused top-k epilogue (one
// translation unit per epilogue so the library compiles in parallel).
#include "fs_stream.h"

namespace fsk {
template hipError_t launch_stream_epi<EPI_TOPK>(const StreamParams&, const StreamConfig&, hipStream_t);
}  // namespace fsk
