// stream_topk.hip -- host-side dispatch of the streaming top-K kernels
// (stream_topk.hpp); the kernels for each list size are instantiated in their
// own translation unit (stream_r*.hip) so they compile in parallel.
#include "stream_topk.hpp"

namespace rt {

// Instantiated in stream_r*.hip (one translation unit per list size and metric).
#define RT_EXTERN_R(R)                                                                                             \
    extern template hipError_t launch_gemv_r<R, false>(bool, int, int, dim3, hipStream_t, const float *, int64_t, \
                                                       int, const float *, const float *, int64_t,                  \
                                                       const TreeLaunch &);                                         \
    extern template hipError_t launch_gemv_r<R, true>(bool, int, int, dim3, hipStream_t, const float *, int64_t,  \
                                                      int, const float *, const float *, int64_t,                   \
                                                      const TreeLaunch &);                                          \
    extern template hipError_t launch_select_r<R>(int, dim3, hipStream_t, const void *, int64_t, int64_t, int64_t, \
                                                  const TreeLaunch &);
RT_EXTERN_R(1)
RT_EXTERN_R(2)
RT_EXTERN_R(4)
RT_EXTERN_R(8)
RT_EXTERN_R(16)
#undef RT_EXTERN_R

bool gemv_fast_path_ok(int d) { return d % 4 == 0 && d / 4 <= 64 * 8; }

int tree_stride(int k, int kp) {
    if (k > kWave / 2) return kp;
    int kc = 1;
    while (kc < k) kc <<= 1;
    return kc;
}

// Pick the lane-group width G = 2^lg (<= 64) and loads per lane L (from
// {1, 2, 3, 4, 6, 8}) that waste the fewest lane slots on a row of d4 16-byte
// blocks, preferring wide groups on ties.
void pick_gemv_shape(int d4, int *log2g, int *L) {
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

template <bool COS>
static hipError_t dispatch_gemv(bool fast, int lg, int L, dim3 grid, hipStream_t s, const float *corpus, int64_t n,
                                int d, const float *queries, const float *rnorm, int64_t per_wave,
                                const TreeLaunch &t) {
    switch (t.kp / 64) {
        case 1: return launch_gemv_r<1, COS>(fast, lg, L, grid, s, corpus, n, d, queries, rnorm, per_wave, t);
        case 2: return launch_gemv_r<2, COS>(fast, lg, L, grid, s, corpus, n, d, queries, rnorm, per_wave, t);
        case 4: return launch_gemv_r<4, COS>(fast, lg, L, grid, s, corpus, n, d, queries, rnorm, per_wave, t);
        case 8: return launch_gemv_r<8, COS>(fast, lg, L, grid, s, corpus, n, d, queries, rnorm, per_wave, t);
        case 16: return launch_gemv_r<16, COS>(fast, lg, L, grid, s, corpus, n, d, queries, rnorm, per_wave, t);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv_topk(const float *corpus, int64_t n, int d, const float *queries, const float *rnorm,
                            int segments, int64_t rows_per_wave, int wgs_per_seg, const TreeLaunch &t,
                            hipStream_t stream) {
    const dim3 grid(wgs_per_seg, segments);
    const bool fast = gemv_fast_path_ok(d);
    int lg = 6, L = 8;
    if (fast) pick_gemv_shape(d / 4, &lg, &L);
    if (rnorm != nullptr)
        return dispatch_gemv<true>(fast, lg, L, grid, stream, corpus, n, d, queries, rnorm, rows_per_wave, t);
    return dispatch_gemv<false>(fast, lg, L, grid, stream, corpus, n, d, queries, nullptr, rows_per_wave, t);
}

hipError_t launch_select_topk(const void *base, int64_t seg_stride, int64_t n, int dtype, int segments,
                              int64_t groups_per_wave, int wgs_per_seg, const TreeLaunch &t, hipStream_t stream) {
    const dim3 grid(wgs_per_seg, segments);
    if (dtype != 0 && dtype != 1) return hipErrorInvalidValue;
    switch (t.kp / 64) {
        case 1: return launch_select_r<1>(dtype, grid, stream, base, n, seg_stride, groups_per_wave, t);
        case 2: return launch_select_r<2>(dtype, grid, stream, base, n, seg_stride, groups_per_wave, t);
        case 4: return launch_select_r<4>(dtype, grid, stream, base, n, seg_stride, groups_per_wave, t);
        case 8: return launch_select_r<8>(dtype, grid, stream, base, n, seg_stride, groups_per_wave, t);
        case 16: return launch_select_r<16>(dtype, grid, stream, base, n, seg_stride, groups_per_wave, t);
        default: return hipErrorInvalidValue;
    }
}

// L2 norm of every corpus row (the per-row norms the cosine metric divides by,
// "GPU-Resident Top-K for Agentic RAG", section 4, Step 2): one wave per row at
// a time, fp64 sum of squares, rounded to fp32 once.
__global__ __launch_bounds__(256) void row_norms_kernel(const float *__restrict__ corpus, int64_t n, int d,
                                                        float *__restrict__ rnorm) {
    const int64_t waves = (int64_t)gridDim.x * (blockDim.x >> 6);
    for (int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave_in_group(); row < n; row += waves) {
        const float v = wave_l2_norm(corpus + row * (int64_t)d, d);
        if (lane_id() == 0) rnorm[row] = v;
    }
}

hipError_t launch_row_norms(const float *corpus, int64_t n, int d, float *rnorm, int num_cus, hipStream_t stream) {
    const int64_t rows_per_block = 4;
    int64_t blocks = (n + rows_per_block - 1) / rows_per_block;
    const int64_t cap = (int64_t)num_cus * 16;
    if (blocks > cap) blocks = cap;
    hipLaunchKernelGGL(row_norms_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, corpus, n, d, rnorm);
    return hipGetLastError();
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
