// filter_r16.hip -- bf16-filtered exact search kernels with 1024-entry lists (see
// filter_topk.hpp).
#include "filter_topk.hpp"

namespace rt {
template hipError_t launch_bound_r<16>(int, int, bool, dim3, hipStream_t, const uint16_t *, int64_t, int,
                                       const float *, const float *, int64_t, const TreeLaunch &,
                                       const FilterLaunch &);
template hipError_t launch_filtered_r<16>(int, int, dim3, hipStream_t, const float *, int64_t, int, const float *,
                                          int64_t, const TreeLaunch &, const FilterLaunch &);
}  // namespace rt
