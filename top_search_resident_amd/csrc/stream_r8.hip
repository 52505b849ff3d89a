// stream_r8.hip -- streaming top-K kernels with 512-entry lists (see stream_topk.hpp).
#include "stream_topk.hpp"

namespace rt {
template hipError_t launch_stream_r<8>(int, int, int, dim3, hipStream_t, const void *, int64_t, int, int64_t,
                                         const float *, int64_t, const TreeLaunch &);
}  // namespace rt
