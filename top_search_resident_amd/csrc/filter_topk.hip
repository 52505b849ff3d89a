// filter_topk.hip -- host-side dispatch of the bf16-filtered exact search
// (filter_topk.hpp) and the bf16 copy of the corpus; the kernels for each list
// size are instantiated in filter_r*.hip.
#include <math.h>

#include "filter_topk.hpp"

namespace rt {

#define RT_EXTERN_F(R)                                                                                             \
    extern template hipError_t launch_bound_r<R>(int, int, bool, dim3, hipStream_t, const uint16_t *, int64_t,    \
                                                 int, const float *, const float *, int64_t, const TreeLaunch &,   \
                                                 const FilterLaunch &);                                            \
    extern template hipError_t launch_filtered_r<R>(int, int, dim3, hipStream_t, const float *, int64_t, int,     \
                                                    const float *, int64_t, const TreeLaunch &, const FilterLaunch &);
RT_EXTERN_F(1)
RT_EXTERN_F(2)
RT_EXTERN_F(4)
RT_EXTERN_F(8)
RT_EXTERN_F(16)
#undef RT_EXTERN_F

bool filtered_search_ok(int d) { return d % 8 == 0 && gemv_fast_path_ok(d); }

float filter_bound_factor(int d) {
    // |a - s| <= |x| |q| (2^-8 + gamma_d (2 + 2^-8)), gamma_d = d u / (1 - d u),
    // u = 2^-24 (2^-8: bf16 rounding; gamma_d: the fp32 sums a and s); then
    // rounded up for the fp32 evaluation of e = cb |q| |x| + delta and of
    // a - e, a + e (a relative 2^-10 covers both with a wide margin).
    const double u = ldexp(1.0, -24);
    const double gamma = d * u / (1.0 - d * u);
    const double c = (ldexp(1.0, -8) + gamma * (2.0 + ldexp(1.0, -8))) * (1.0 + ldexp(1.0, -10));
    return nextafterf((float)c, INFINITY);
}

float filter_underflow_slack(int d) {
    // Values below 2^-126 round to bf16 with an absolute error of at most
    // 2^-134 (|q|_1 <= sqrt(d) |q| of it), and each of the 2d fused
    // multiply-adds of the two sums loses at most 2^-126 to underflow even when
    // results below 2^-126 are flushed: 3 d 2^-126 max(|q|, 1) covers both;
    // 4 d 2^-126 leaves room for rounding e.
    return ldexpf((float)d, -124);
}

hipError_t launch_filtered_search(const float *corpus, const uint16_t *corpus16, const float *rnorm, int64_t n,
                                  int d, const float *queries, int segments, int64_t rows_per_wave1, int wgs1,
                                  const TreeLaunch &t1, int64_t rows_per_wave2, int wgs2, const TreeLaunch &t2,
                                  const FilterLaunch &f, hipEvent_t between, hipStream_t stream) {
    if (!filtered_search_ok(d)) return hipErrorInvalidValue;
    int lg8 = 6, L8 = 8, lg4 = 6, L4 = 8;
    pick_gemv_shape(d / 8, &lg8, &L8);
    pick_gemv_shape(d / 4, &lg4, &L4);
    const bool ahead = rows_per_wave1 <= kGemvLookaheadRows;
    const dim3 g1(wgs1, segments), g2(wgs2, segments);
    hipError_t err;
    switch (t1.kp / 64) {
        case 1: err = launch_bound_r<1>(lg8, L8, ahead, g1, stream, corpus16, n, d, queries, rnorm, rows_per_wave1, t1, f); break;
        case 2: err = launch_bound_r<2>(lg8, L8, ahead, g1, stream, corpus16, n, d, queries, rnorm, rows_per_wave1, t1, f); break;
        case 4: err = launch_bound_r<4>(lg8, L8, ahead, g1, stream, corpus16, n, d, queries, rnorm, rows_per_wave1, t1, f); break;
        case 8: err = launch_bound_r<8>(lg8, L8, ahead, g1, stream, corpus16, n, d, queries, rnorm, rows_per_wave1, t1, f); break;
        case 16: err = launch_bound_r<16>(lg8, L8, ahead, g1, stream, corpus16, n, d, queries, rnorm, rows_per_wave1, t1, f); break;
        default: return hipErrorInvalidValue;
    }
    if (err != hipSuccess) return err;
    if (between) err = hipEventRecord(between, stream);
    if (err != hipSuccess) return err;
    switch (t2.kp / 64) {
        case 1: return launch_filtered_r<1>(lg4, L4, g2, stream, corpus, n, d, queries, rows_per_wave2, t2, f);
        case 2: return launch_filtered_r<2>(lg4, L4, g2, stream, corpus, n, d, queries, rows_per_wave2, t2, f);
        case 4: return launch_filtered_r<4>(lg4, L4, g2, stream, corpus, n, d, queries, rows_per_wave2, t2, f);
        case 8: return launch_filtered_r<8>(lg4, L4, g2, stream, corpus, n, d, queries, rows_per_wave2, t2, f);
        case 16: return launch_filtered_r<16>(lg4, L4, g2, stream, corpus, n, d, queries, rows_per_wave2, t2, f);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_filtered_pass2(const float *corpus, int64_t n, int d, const float *queries, int segments,
                                 int64_t rows_per_wave, int wgs, const TreeLaunch &t, const FilterLaunch &f,
                                 hipStream_t stream) {
    if (!filtered_search_ok(d)) return hipErrorInvalidValue;
    int lg4 = 6, L4 = 8;
    pick_gemv_shape(d / 4, &lg4, &L4);
    const dim3 g(wgs, segments);
    switch (t.kp / 64) {
        case 1: return launch_filtered_r<1>(lg4, L4, g, stream, corpus, n, d, queries, rows_per_wave, t, f);
        case 2: return launch_filtered_r<2>(lg4, L4, g, stream, corpus, n, d, queries, rows_per_wave, t, f);
        case 4: return launch_filtered_r<4>(lg4, L4, g, stream, corpus, n, d, queries, rows_per_wave, t, f);
        case 8: return launch_filtered_r<8>(lg4, L4, g, stream, corpus, n, d, queries, rows_per_wave, t, f);
        case 16: return launch_filtered_r<16>(lg4, L4, g, stream, corpus, n, d, queries, rows_per_wave, t, f);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_filtered_collect(const float *corpus, int64_t n, int d, const float *queries, int segments,
                                   int64_t rows_per_wave, int wgs, const TreeLaunch &t, const FilterLaunch &f,
                                   hipStream_t stream) {
    if (!filtered_search_ok(d) || f.cand == nullptr || f.cand_cnt == nullptr || f.cand_ld < n ||
        f.cnt_ld < (int64_t)wgs * collect_waves() || t.k > 64)
        return hipErrorInvalidValue;
    int lg4 = 6, L4 = 8;
    pick_gemv_shape(d / 4, &lg4, &L4);
    // 64-entry list instantiations: in collect mode the selectors are idle
    return launch_filtered_r<1>(lg4, L4, dim3(wgs, segments), stream, corpus, n, d, queries, rows_per_wave, t, f);
}

// Round to nearest even; a value that is not finite or rounds to infinity is
// reported through *bad (its copy is then unusable for bounds).
__global__ __launch_bounds__(256) void to_bf16_kernel(const float *__restrict__ x, uint16_t *__restrict__ y,
                                                      int64_t count, uint32_t *bad) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    uint32_t flag = 0;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
        const uint32_t b = __float_as_uint(x[i]);
        const uint32_t r = b + 0x7fffu + ((b >> 16) & 1u);
        if ((b & 0x7f800000u) == 0x7f800000u || (r & 0x7f800000u) == 0x7f800000u) flag = 1;
        y[i] = (uint16_t)(r >> 16);
    }
    if (__ballot(flag != 0) != 0 && lane_id() == 0) atomicOr(bad, 1u);
}

// err[row] >= || x - bf16(x) || for every row x (bf16 as to_bf16_kernel rounds):
// each difference is exact in fp32 (the bits that rounding drops) and its
// square exact in fp64; the fp64 sum (error <= d 2^-53 relative) and square
// root are rounded up by a relative 2^-40 and then to fp32 upward, so the value
// is never below the true norm.  One wave per row; a value that overflows in
// bf16 leaves the copy unusable anyway (to_bf16_kernel's flag).
__global__ __launch_bounds__(256) void bf16_row_error_kernel(const float *__restrict__ corpus, int64_t n, int d,
                                                             float *__restrict__ err) {
    const int64_t waves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int lane = lane_id();
    for (int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave_in_group(); row < n; row += waves) {
        const float *v = corpus + row * (int64_t)d;
        double s = 0.0;
        for (int c = lane; c < d; c += 64) {
            const float x = v[c];
            const uint32_t b = __float_as_uint(x);
            const float xb = __uint_as_float(((b + 0x7fffu + ((b >> 16) & 1u)) >> 16) << 16);
            const double e = (double)x - (double)xb;
            s = fma(e, e, s);
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
        if (lane == 0) {
            const double up = sqrt(s) * (1.0 + 0x1p-40);
            float f = (float)up;
            if ((double)f < up) f = __uint_as_float(__float_as_uint(f) + 1u);  // next fp32 up (f >= 0)
            err[row] = f;
        }
    }
}

hipError_t launch_bf16_row_errors(const float *corpus, int64_t n, int d, float *err, int num_cus,
                                  hipStream_t stream) {
    int64_t blocks = (n + 3) / 4;
    const int64_t cap = (int64_t)num_cus * 16;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(bf16_row_error_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, corpus, n, d, err);
    return hipGetLastError();
}

hipError_t launch_to_bf16(const float *corpus, uint16_t *corpus16, int64_t count, uint32_t *bad, int num_cus,
                          hipStream_t stream) {
    int64_t blocks = (count + 255) / 256;
    const int64_t cap = (int64_t)num_cus * 32;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(to_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, corpus, corpus16, count, bad);
    return hipGetLastError();
}

}  // namespace rt
