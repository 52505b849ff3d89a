// stream_r1c.hip -- cosine scoring kernels with 64-entry lists (see
// stream_topk.hpp).
#include "stream_topk.hpp"

namespace rt {
template hipError_t launch_gemv_r<1, true>(bool, int, int, dim3, hipStream_t, const float *, int64_t, int,
                                          const float *, const float *, int64_t, const TreeLaunch &);
}  // namespace rt
