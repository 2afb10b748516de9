// fs_stream_flat.hip -- streaming kernels with the flat epilogue (one
// translation unit per epilogue so the library compiles in parallel).
#include "fs_stream.h"

namespace fsk {
template hipError_t launch_stream_epi<EPI_FLAT>(const StreamParams&, const StreamConfig&, hipStream_t);
}  // namespace fsk
