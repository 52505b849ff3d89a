// stream_r8.hip -- inner-product scoring and raw-array selection kernels with
// 512-entry lists (see stream_topk.hpp).
#include "stream_topk.hpp"

namespace rt {
template hipError_t launch_gemv_r<8, false>(bool, int, int, dim3, hipStream_t, const float *, int64_t, int,
                                           const float *, const float *, int64_t, const TreeLaunch &);
template hipError_t launch_select_r<8>(int, dim3, hipStream_t, const void *, int64_t, int64_t, int64_t,
                                        const TreeLaunch &);
}  // namespace rt
