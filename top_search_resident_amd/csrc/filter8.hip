// filter8.hip -- the fp8 copy of the corpus and the filtered search's first
// pass over it (filter8.hpp); the second pass is the bf16 path's.
#include <math.h>

#include "filter8.hpp"
#include "filter8_host.hpp"

namespace rt {

// Depths with an fp8 first pass and their lane-group shapes X(d16, LG, L, P)
// over 16-byte blocks (d16 = d / 16 = G L exactly), P steps of loads in flight:
// about 4 KB of codes per wave step, four blocks per lane where four divide the
// row, else three, two steps ahead (measured on MI355X at 2^30 elements, pass 1
// at K = 8 against whole-row groups of one or two blocks four steps ahead:
// d = 1024 172.7 against 193.1 us, 512 191.5 against 205.3, 768 184.4 against
// 186.3, 2048 184.9 against 182.8); rows of 256 keep 16-lane groups of one
// block, two rows per step four steps ahead (212.6 us against 230.4 for 4-lane
// groups of four blocks).
#define RT_FP8_SHAPES(X) \
    X(16, 4, 1, 4) X(24, 3, 3, 2) X(32, 3, 4, 2) X(48, 4, 3, 2) X(64, 4, 4, 2) X(96, 5, 3, 2) X(128, 5, 4, 2)

bool fp8_search_ok(int d) {
    return d == 256 || d == 384 || d == 512 || d == 768 || d == 1024 || d == 1536 || d == 2048;
}

void filter_bound_constants_fp8(int d, float *cr, float *cx, float *delta) {
    const double u = ldexp(1.0, -24);
    const double gamma = d * u / (1.0 - d * u);
    const double slack = 1.0 + ldexp(1.0, -10);
    *cr = nextafterf((float)((1.0 + gamma) * slack), INFINITY);
    *cx = nextafterf((float)(2.0 * gamma * slack), INFINITY);
    *delta = ldexpf((float)d, -124);
}

// One wave per row: s = the power of two with max |x| <= 224 s (s >= 2^-126;
// 1 for a zero row), codes = e4m3 of x / s (the hardware conversion), and
// meta = {s, c}, c >= cr err + cx rnorm[row] (rounded up), err >= |x - s
// dec(codes)| from the stored codes themselves (fp64 sum of squares of exact
// differences, square root rounded up by 2^-40).  A value that is not finite
// sets *bad.  Lane l converts elements 16 l .. 16 l + 15 of each 1024-element
// chunk (d % 16 == 0).
__global__ __launch_bounds__(256) void to_fp8_kernel(const float *__restrict__ corpus, int64_t n, int d,
                                                     const float *__restrict__ rnorm, float cr, float cx,
                                                     uint8_t *__restrict__ codes, float2 *__restrict__ meta,
                                                     uint32_t *bad) {
    const int64_t waves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int lane = lane_id();
    uint32_t flag = 0;
    for (int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave_in_group(); row < n; row += waves) {
        const float *v = corpus + row * (int64_t)d;
        float mx = 0.f;
        for (int c = lane; c < d; c += 64) {
            const float x = v[c];
            if (!(fabsf(x) <= __FLT_MAX__)) flag = 1;
            mx = fmaxf(mx, fabsf(x));
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
        // smallest k with mx <= 224 2^k: mx = f 2^e, f in [0.5, 1), 224 = 0.875 2^8
        int e = 0;
        const float f = frexpf(mx, &e);
        int k = (f <= 0.875f) ? e - 8 : e - 7;
        if (mx == 0.f || !(mx <= __FLT_MAX__)) k = 0;
        k = k < -126 ? -126 : k;
        const float s = ldexpf(1.f, k);
        const float inv = ldexpf(1.f, -k);
        double ss = 0.0;
        uint8_t *out = codes + row * (int64_t)d;
        for (int c0 = 16 * lane; c0 < d; c0 += 1024) {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x0 = v[c0 + 4 * i], x1 = v[c0 + 4 * i + 1];
                const float x2 = v[c0 + 4 * i + 2], x3 = v[c0 + 4 * i + 3];
                int p = __builtin_amdgcn_cvt_pk_fp8_f32(x0 * inv, x1 * inv, 0, false);
                p = __builtin_amdgcn_cvt_pk_fp8_f32(x2 * inv, x3 * inv, p, true);
                w[i] = (uint32_t)p;
                const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(p, false);
                const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(p, true);
                const double d0 = (double)x0 - (double)lo[0] * (double)s;
                const double d1 = (double)x1 - (double)lo[1] * (double)s;
                const double d2 = (double)x2 - (double)hi[0] * (double)s;
                const double d3 = (double)x3 - (double)hi[1] * (double)s;
                ss = fma(d0, d0, ss);
                ss = fma(d1, d1, ss);
                ss = fma(d2, d2, ss);
                ss = fma(d3, d3, ss);
            }
            *reinterpret_cast<uint4 *>(out + c0) = make_uint4(w[0], w[1], w[2], w[3]);
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
        if (lane == 0) {
            // each fp64 step below rounds by at most 2^-53 relative: 2^-40 covers them
            const double up = ((double)cr * (sqrt(ss) * (1.0 + 0x1p-40)) + (double)cx * (double)rnorm[row]) *
                              (1.0 + 0x1p-40);
            float c = (float)up;
            if ((double)c < up) c = __uint_as_float(__float_as_uint(c) + 1u);  // next fp32 up (c >= 0)
            meta[row] = make_float2(s, c);
        }
    }
    if (__ballot(flag != 0) != 0 && lane == 0) atomicOr(bad, 1u);
}

hipError_t launch_to_fp8(const float *corpus, int64_t n, int d, const float *rnorm, uint8_t *codes, float2 *meta,
                         uint32_t *bad, int num_cus, hipStream_t stream) {
    float cr = 0.f, cx = 0.f, delta = 0.f;
    filter_bound_constants_fp8(d, &cr, &cx, &delta);
    int64_t blocks = (n + 3) / 4;
    const int64_t cap = (int64_t)num_cus * 16;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(to_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, corpus, n, d, rnorm, cr, cx,
                       codes, meta, bad);
    return hipGetLastError();
}

template <int R>
static hipError_t launch_bound8_r(dim3 grid, hipStream_t s, const Fp8Rows &fr, int64_t n, int d,
                                  const float *queries, int64_t per_wave, const TreeLaunch &t, const FilterLaunch &f) {
    const TreeArgs ta = make_tree(t);
    const FilterArgs fa = make_filter(f);
    const dim3 block(64 * gemv_waves(64 * R));
#define RT_SHAPE8(D16, LGV, LV, PV)                                                                              \
    static_assert((1 << LGV) * LV == D16, "an fp8 shape covers its row exactly");                                \
    if (d == 16 * D16) {                                                                                         \
        if (fa.crn)                                                                                              \
            hipLaunchKernelGGL((gemv_bound8_kernel<LGV, LV, R, PV, true>), grid, block, 0, s, fr, n, d, queries, \
                               per_wave, ta, fa);                                                                \
        else                                                                                                     \
            hipLaunchKernelGGL((gemv_bound8_kernel<LGV, LV, R, PV, false>), grid, block, 0, s, fr, n, d,         \
                               queries, per_wave, ta, fa);                                                       \
        return hipGetLastError();                                                                                \
    }
    RT_FP8_SHAPES(RT_SHAPE8)
#undef RT_SHAPE8
    return hipErrorInvalidValue;
}

hipError_t launch_filtered_search8(const float *corpus, const uint8_t *codes, const float2 *meta, int64_t n, int d,
                                   const float *queries, int segments, int64_t rows_per_wave1, int wgs1,
                                   const TreeLaunch &t1, int64_t rows_per_wave2, int wgs2, const TreeLaunch &t2,
                                   const FilterLaunch &f, hipEvent_t between, hipStream_t stream) {
    if (!fp8_search_ok(d)) return hipErrorInvalidValue;
    Fp8Rows fr;
    fr.codes = codes;
    fr.meta = meta;
    float cr = 0.f, cx = 0.f;
    filter_bound_constants_fp8(d, &cr, &cx, &fr.delta);
    const dim3 g1(wgs1, segments);
    hipError_t err;
    switch (t1.kp / 64) {
        case 1: err = launch_bound8_r<1>(g1, stream, fr, n, d, queries, rows_per_wave1, t1, f); break;
        case 2: err = launch_bound8_r<2>(g1, stream, fr, n, d, queries, rows_per_wave1, t1, f); break;
        case 4: err = launch_bound8_r<4>(g1, stream, fr, n, d, queries, rows_per_wave1, t1, f); break;
        case 8: err = launch_bound8_r<8>(g1, stream, fr, n, d, queries, rows_per_wave1, t1, f); break;
        case 16: err = launch_bound8_r<16>(g1, stream, fr, n, d, queries, rows_per_wave1, t1, f); break;
        default: return hipErrorInvalidValue;
    }
    if (err != hipSuccess) return err;
    if (between) err = hipEventRecord(between, stream);
    if (err != hipSuccess) return err;
    return launch_filtered_pass2(corpus, n, d, queries, segments, rows_per_wave2, wgs2, t2, f, stream);
}

}  // namespace rt
