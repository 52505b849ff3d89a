// filter8_host.hpp -- host-side launchers of the fp8 first pass (filter8.hip),
// internal to libresident_topk.
#pragma once
#include "kernels.hpp"

namespace rt {

// Depths with an fp8 first pass (d / 16 blocks of codes per row).
bool fp8_search_ok(int d);
// e = |q| (cr |x - x~| + cx |x|) + delta max(|q|, 1) max(s, 1) for depth d.
void filter_bound_constants_fp8(int d, float *cr, float *cx, float *delta);
// codes = e4m3 of each row / its power-of-two scale s, meta[row] = {s, c} with
// c >= cr |row - s dec(codes)| + cx rnorm[row], for rows < n (d % 16 == 0);
// *bad set if a value is not finite (the caller clears it).
hipError_t launch_to_fp8(const float *corpus, int64_t n, int d, const float *rnorm, uint8_t *codes, float2 *meta,
                         uint32_t *bad, int num_cus, hipStream_t stream);
// Both passes of the filtered search with the fp8 first pass; grids (wgs1 or
// wgs2, segments); `between` (may be null) is recorded after pass 1.
hipError_t launch_filtered_search8(const float *corpus, const uint8_t *codes, const float2 *meta, int64_t n, int d,
                                   const float *queries, int segments, int64_t rows_per_wave1, int wgs1,
                                   const TreeLaunch &t1, int64_t rows_per_wave2, int wgs2, const TreeLaunch &t2,
                                   const FilterLaunch &f, hipEvent_t between, hipStream_t stream);

}  // namespace rt
