// stream_topk.hip -- host-side dispatch of the streaming top-K kernels
// (stream_topk.hpp); the kernels for each list size are instantiated in their
// own translation unit (stream_r*.hip) so they compile in parallel.
#include "stream_topk.hpp"

namespace rt {

template <int R>
hipError_t launch_stream_r(int kind, int lg, int L, dim3 grid, hipStream_t s, const void *data, int64_t n, int d,
                           int64_t seg_stride, const float *queries, int64_t per_wave, const TreeLaunch &t);

bool gemv_fast_path_ok(int d) { return d % 4 == 0 && d / 4 <= 64 * 8; }

int tree_fan(int kp) { return kTreeEntries / kp; }

// Pick the lane-group width G = 2^lg (<= 64) and loads per lane L (from
// {1, 2, 3, 4, 6, 8}) that waste the fewest lane slots on a row, preferring wide
// groups on ties.
static void pick_group(int d4, int *log2g, int *L) {
    static const int Ls[6] = {1, 2, 3, 4, 6, 8};
    int best_waste = 1 << 30, best_lg = 6, best_L = 8;
    for (int lg = 6; lg >= 0; --lg) {
        const int G = 1 << lg;
        for (int i = 0; i < 6; ++i) {
            if (G * Ls[i] < d4) continue;
            const int waste = G * Ls[i] - d4;
            if (waste < best_waste) {
                best_waste = waste;
                best_lg = lg;
                best_L = Ls[i];
            }
            break;
        }
    }
    *log2g = best_lg;
    *L = best_L;
}

static hipError_t dispatch(int kind, int lg, int L, dim3 grid, hipStream_t s, const void *data, int64_t n, int d,
                           int64_t seg_stride, const float *queries, int64_t per_wave, const TreeLaunch &t) {
    switch (t.kp / 64) {
        case 1: return launch_stream_r<1>(kind, lg, L, grid, s, data, n, d, seg_stride, queries, per_wave, t);
        case 2: return launch_stream_r<2>(kind, lg, L, grid, s, data, n, d, seg_stride, queries, per_wave, t);
        case 4: return launch_stream_r<4>(kind, lg, L, grid, s, data, n, d, seg_stride, queries, per_wave, t);
        case 8: return launch_stream_r<8>(kind, lg, L, grid, s, data, n, d, seg_stride, queries, per_wave, t);
        case 16: return launch_stream_r<16>(kind, lg, L, grid, s, data, n, d, seg_stride, queries, per_wave, t);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv_topk(const float *corpus, int64_t n, int d, const float *queries, int segments,
                            int64_t rows_per_wave, int wgs_per_seg, const TreeLaunch &t, hipStream_t stream) {
    const dim3 grid(wgs_per_seg, segments);
    if (!gemv_fast_path_ok(d)) return dispatch(1, 0, 0, grid, stream, corpus, n, d, 0, queries, rows_per_wave, t);
    int lg = 6, L = 8;
    pick_group(d / 4, &lg, &L);
    return dispatch(0, lg, L, grid, stream, corpus, n, d, 0, queries, rows_per_wave, t);
}

hipError_t launch_select_topk(const void *base, int64_t seg_stride, int64_t n, int dtype, int segments,
                              int64_t groups_per_wave, int wgs_per_seg, const TreeLaunch &t, hipStream_t stream) {
    const dim3 grid(wgs_per_seg, segments);
    if (dtype != 0 && dtype != 1) return hipErrorInvalidValue;
    return dispatch(2 + dtype, 0, 0, grid, stream, base, n, 0, seg_stride, nullptr, groups_per_wave, t);
}

__global__ void zero_u32_kernel(uint32_t *p, int64_t count) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) p[i] = 0u;
}

hipError_t launch_zero_counters(uint32_t *counters, int64_t count, hipStream_t stream) {
    hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream, counters, count);
    return hipGetLastError();
}

}  // namespace rt
