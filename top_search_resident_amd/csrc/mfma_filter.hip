// mfma_filter.hip -- exact batched inner-product top-K through the bf16 copy of
// the corpus, on CDNA4 matrix cores (gfx950).
//
// The plain batch (mfma_scores.hip) reads the fp32 corpus once for up to 32
// queries and multiplies on v_mfma_f32_32x32x2_f32.  Here the first pass reads
// the bf16 copy instead (half the bytes) and multiplies on
// v_mfma_f32_32x32x16_bf16, whose arithmetic is small next to the bytes.  As in
// the single-query filtered search (filter_topk.hpp; the pages' plan of
// reduced-precision storage with a full-precision re-rank of the candidates,
// "CUDA Programming Model Series 9: Efficient TopK" section 4.3, and the third
// stage, re-rank and output, of the BANG page "how BANG achieves billion-scale
// ANN search with GPU micro-kernels"), the first pass may only exclude rows it
// can prove are not in the answer:
//
//   pass 1 (mfma_bound_kernel): for query j and row i, a = the bf16 MFMA sum of
//     bf16(x_i) against the query split into two bf16 parts (q = hi + lo + r,
//     |r| <= 2^-16 |q|), a bound e with |a - s| <= e, where s is the score the
//     plain single-query scan computes in fp32, the upper bound a + e stored
//     per (query, row), and per query the largest lower bound a - e of every
//     32-row tile;
//   pass 1b (tile_threshold_kernel, batch_select.hip): per query T = the lower
//     edge of a key bin holding the k-th largest of those tile maxima.  k tiles
//     reach T, each holds a row whose lower bound reaches T, so k rows have
//     s >= T: every row of the top k has s >= T and therefore an upper bound
//     >= T;
//   pass 2 (gemv_filtered_kernel, filter_topk.hpp): per query, only the rows
//     whose upper bound reaches T are re-scored from the fp32 corpus with the
//     plain scan's arithmetic and selected.
// So each query's answer is the plain single-query scan's answer, bit for bit.
//
// The bound (host: filter_bound_constants_batched).  With x~ = bf16(x),
// q' = hi + lo, P = sum x q and A = sum x~ q' (exact), and u = 2^-24:
//   |A - P| <= |x~ - x| |q'| + 2^-16 |x| |q|  (Cauchy-Schwarz on the rounding
//              error vector; |q'| <= (1 + 2^-16) |q|),
//   |a - A| <= 1.02 g |x| |q|, g = 8 d u / (1 - 8 d u): the matrix core's fp32
//              accumulation of the 2 d exact products in any order and
//              rounding direction allows 4 d u on sum |x~| (|hi| + |lo|) <=
//              1.02 |x| |q|; the factor 2 leaves room for alignment inside
//              the unit,
//   |P - s| <= gamma_d |x| |q|, gamma_d = d u / (1 - d u) (the plain scan),
// so e = |q| (cr |x~ - x| + cx |x|) + delta max(|q|, 1) max(|x|, 1) with
// cr = (1 + 2^-16) and cx = 2^-16 + gamma_d + 1.02 g, both times (1 + 2^-10)
// and rounded up (the 2^-10 absorbs the fp32 evaluation of e and a +- e), and
// delta = 16 d 2^-126 for values, products and partial sums below 2^-126
// whether the unit flushes them or not.  |x~ - x| per row is computed once with
// the bf16 copy, rounded up (bf16_row_error_kernel); for rows of Gaussian
// entries it is about 0.4 2^-8 |x|, against 2^-8 |x| for the elementwise
// worst case.  A sum or bound that is not finite gives the row the bounds
// -inf and +inf.
#include <math.h>

#include <utility>

#include "filter_topk.hpp"

namespace rt {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Round to nearest even (the rounding of the corpus copy, to_bf16_kernel).
__device__ __forceinline__ uint32_t bf16_bits_rne(float x) {
    const uint32_t b = __float_as_uint(x);
    return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), so that
// ring-slot indices are compile-time constants.
template <typename F, int... I>
__device__ __forceinline__ void bound_static_for_seq(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void bound_static_for(F &&f) {
    bound_static_for_seq(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ float comp4(const float4 &v, int c) {
    return c == 0 ? v.x : (c == 1 ? v.y : (c == 2 ? v.z : v.w));
}

// Pass 1 for d = 64 NCK.  One workgroup per CU holds the 32 x d query block as
// bf16 hi and lo parts in LDS (row stride d + 8 bf16, so the 32 lanes reading
// one column of the block hit distinct banks), then a 4 KB staging buffer per
// wave.  A wave computes 32-row tiles, 64 columns (128 bytes of a bf16 row) at
// a time: load instruction i (0..3) gives lane l the 16 bytes at row 8 i + l / 8,
// byte 16 (l % 8) of the chunk -- 8 rows x 128 contiguous bytes per
// instruction -- which the wave writes to its staging buffer and reads back in
// the MFMA layout: for k-step s (0..3), lane (m = l % 32, h = l / 32) takes row
// m's 16-byte unit 2 s + h, and its query operand is query m's same 8 columns,
// so the MFMA's k-slots pair corpus and query columns exactly (hi and lo parts:
// two MFMAs per k-step).  Unit u of staged row r sits at position u ^ f(r),
// f(r) = (r ^ (r >> 3)) & 7, so neither the row-wise writes nor the column-wise
// reads collide in LDS banks.  Only the wave's own lanes exchange data through
// its buffer (no workgroup barrier).  Global loads run KPF chunks ahead of the
// chunk being staged, across the wave's consecutive tiles; a chunk is staged
// and its operands read while the previous chunk's MFMAs run.  The output tile
// (rows x queries) has row 8 g + 4 h + c, query m in register 4 g + c of lane
// m + 32 h.
__device__ __forceinline__ int bound_swizzle(int r) { return (r ^ (r >> 3)) & 7; }

template <int NCK, int NW, int KPF>
__global__ __launch_bounds__(NW * 64) void mfma_bound_kernel(const uint16_t *__restrict__ corpus16, int64_t n,
                                                            const float *__restrict__ queries, int q,
                                                            const float *__restrict__ rnorm,
                                                            const float *__restrict__ rerr, float cr, float cx,
                                                            float delta, float *__restrict__ ubuf, int64_t uld,
                                                            float *__restrict__ tlb, int64_t tld,
                                                            int64_t tiles_per_wave) {
    static_assert(KPF >= 1 && KPF < NCK && NCK % KPF == 0, "pipeline shape");
    constexpr int d = NCK * 64;
    constexpr int dp = d + 8;
    constexpr int d16 = d / 8;  // 16-byte units per row
    // [2][32][dp] bf16 query parts (hi, then lo), then NW staging buffers of 256 x 16 bytes
    extern __shared__ __align__(16) uint16_t qbf[];
    __shared__ float qn_s[kMfmaMaxQ];
    uint16_t *const qh = qbf;
    uint16_t *const ql = qbf + kMfmaMaxQ * dp;
    for (int i = threadIdx.x; i < kMfmaMaxQ * d; i += NW * 64) {
        const int r = i / d, c = i - r * d;
        const float x = (r < q) ? queries[(int64_t)r * d + c] : 0.f;
        const uint32_t hb = bf16_bits_rne(x);
        qh[r * dp + c] = (uint16_t)hb;
        ql[r * dp + c] = (uint16_t)bf16_bits_rne(x - __uint_as_float(hb << 16));
    }
    for (int j = wave_in_group(); j < kMfmaMaxQ; j += NW) {
        const float v = (j < q) ? wave_l2_norm(queries + (int64_t)j * d, d) : 0.f;
        if (lane_id() == 0) qn_s[j] = v;
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int wv = wave_in_group();
    const int m = lane & 31;
    const int h = lane >> 5;
    const int rsub = lane >> 3;  // row within a load instruction's 8 rows
    const int unit = lane & 7;   // 16-byte unit within the chunk
    const float qn = qn_s[m];
    const float er = cr * qn;
    const float ex = cx * qn;
    const float dl = delta * fmaxf(qn, 1.f);
    const bool has_q = m < q;
    const int64_t wave = (int64_t)blockIdx.x * NW + wv;
    const int64_t tiles = (n + 31) / 32;
    const int64_t t_begin = wave * tiles_per_wave;
    const int64_t t_end = (t_begin + tiles_per_wave < tiles) ? t_begin + tiles_per_wave : tiles;
    if (t_begin >= t_end) return;  // no barrier follows

    uint4 *const stage = reinterpret_cast<uint4 *>(qbf + 2 * kMfmaMaxQ * dp) + wv * 256;
    const int fm = bound_swizzle(m);
    const uint4 *__restrict__ c16 = reinterpret_cast<const uint4 *>(corpus16);
    // 16-byte offsets of this lane's four rows of tile tt (rows past n read row n - 1)
    struct Rows {
        int64_t o[4];
    };
    auto rows_of = [&](int64_t tt) {
        Rows r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t row = tt * 32 + 8 * i + rsub;
            r.o[i] = (row < n ? row : n - 1) * (int64_t)d16 + unit;
        }
        return r;
    };
    auto gload = [&](const Rows &r, int chunk, uint4(&dst)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = load_nt(c16 + r.o[i] + chunk * 8);
    };
    auto stage_store = [&](const uint4(&src)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) stage[(8 * i + rsub) * 8 + (unit ^ rsub ^ i)] = src[i];
    };
    auto stage_load = [&](uint4(&dst)[4]) {
#pragma unroll
        for (int s = 0; s < 4; ++s) dst[s] = stage[m * 8 + ((2 * s + h) ^ fm)];
    };
    auto qload = [&](const uint16_t *base, int chunk, uint4(&dst)[4]) {
#pragma unroll
        for (int s = 0; s < 4; ++s) dst[s] = *reinterpret_cast<const uint4 *>(base + chunk * 64 + 16 * s);
    };

    int64_t t = t_begin;
    Rows pc = rows_of(t);
    Rows pn = rows_of(t + 1 < t_end ? t + 1 : t);  // past the wave's last tile: reload (cached)
    uint4 g[KPF][4];
#pragma unroll
    for (int s = 0; s < KPF; ++s) gload(pc, s, g[s]);
    uint4 acur[4], bhc[4], blc[4];
    stage_store(g[0]);
    wave_lds_sync();
    stage_load(acur);
    qload(qh + m * dp + 8 * h, 0, bhc);
    qload(ql + m * dp + 8 * h, 0, blc);
    gload(pc, KPF, g[0]);
    for (;;) {
        // Opaque per-tile offset: keeps the compiler from hoisting every
        // chunk's query operands into registers.
        int qoff = 0;
        asm volatile("" : "+v"(qoff));
        const uint16_t *qhr = qh + m * dp + 8 * h + qoff;
        const uint16_t *qlr = ql + m * dp + 8 * h + qoff;
        float4 rn[4], re[4];
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            rn[gg] = *reinterpret_cast<const float4 *>(rnorm + t * 32 + 4 * h + 8 * gg);
            re[gg] = *reinterpret_cast<const float4 *>(rerr + t * 32 + 4 * h + 8 * gg);
        }
        floatx16 acc;
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] = 0.f;
        bound_static_for<NCK>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            // Stage chunk j + 1 (the next tile's chunk 0 after the last) from
            // its ring slot, read its operands, refill the slot, then multiply
            // chunk j.
            constexpr int sn = (j + 1) % KPF;
            constexpr int jn = (j + 1 < NCK) ? j + 1 : 0;
            uint4 anext[4], bhn[4], bln[4];
            stage_store(g[sn]);
            wave_lds_sync();
            stage_load(anext);
            qload(qhr, jn, bhn);
            qload(qlr, jn, bln);
            if constexpr (j + 1 + KPF < NCK)
                gload(pc, j + 1 + KPF, g[sn]);
            else
                gload(pn, j + 1 + KPF - NCK, g[sn]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 a = __builtin_bit_cast(bf16x8, acur[s]);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, bhc[s]), acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, blc[s]), acc, 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                acur[s] = anext[s];
                bhc[s] = bhn[s];
                blc[s] = bln[s];
            }
        });
        // Bounds of the tile's rows for query m; upper bounds stored, the
        // tile's largest lower bound kept.
        float mx = -__builtin_huge_valf();
        float *urow = ubuf + (int64_t)m * uld + t * 32 + 4 * h;
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            const int64_t r = t * 32 + 8 * gg + 4 * h;
            float ubv[4], lbv[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float a = acc[4 * gg + c];
                const float rv = comp4(rn[gg], c);
                const float e = fmaf(er, comp4(re[gg], c), fmaf(ex, rv, dl * fmaxf(rv, 1.f)));
                // false for an overflowed or NaN sum or bound: the row is kept
                const bool known = fabsf(a) <= __FLT_MAX__ && e <= __FLT_MAX__;
                ubv[c] = known ? a + e : __builtin_huge_valf();
                lbv[c] = known ? a - e : -__builtin_huge_valf();
            }
            if (r + 3 < n) {
                if (has_q) *reinterpret_cast<float4 *>(urow + 8 * gg) = make_float4(ubv[0], ubv[1], ubv[2], ubv[3]);
                mx = fmaxf(mx, fmaxf(fmaxf(lbv[0], lbv[1]), fmaxf(lbv[2], lbv[3])));
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if (r + c < n) {
                        if (has_q) urow[8 * gg + c] = ubv[c];
                        mx = fmaxf(mx, lbv[c]);
                    }
                }
            }
        }
        mx = fmaxf(mx, __uint_as_float(xor_u32<32>(__float_as_uint(mx))));
        if (h == 0 && has_q) tlb[(int64_t)m * tld + t] = mx;
        if (t + 1 >= t_end) break;
        ++t;
        pc = pn;
        pn = rows_of(t + 1 < t_end ? t + 1 : t);
    }
}

bool mfma_filter_ok(int d) { return d == 256 || d == 384 || d == 512 || d == 768 || d == 1024; }

void filter_bound_constants_batched(int d, float *cr, float *cx, float *delta) {
    const double u = ldexp(1.0, -24);
    const double gamma = d * u / (1.0 - d * u);
    const double g8 = 8.0 * d * u / (1.0 - 8.0 * d * u);
    const double slack = 1.0 + ldexp(1.0, -10);
    *cr = nextafterf((float)((1.0 + ldexp(1.0, -16)) * slack), INFINITY);
    *cx = nextafterf((float)((ldexp(1.0, -16) + gamma + 1.02 * g8) * slack), INFINITY);
    *delta = ldexpf((float)d, -122);
}

// Pass 1's shapes: (chunks NCK = d / 64, waves per workgroup NW, chunks in
// flight per wave KPF).  One workgroup per CU; NW is what the LDS holds next to
// the query block (7 at d = 1024), KPF divides NCK.
#define RT_BOUND_DEPTHS(X) X(4, 8, 2) X(6, 8, 3) X(8, 8, 4) X(12, 8, 4) X(16, 7, 4)

static size_t bound_lds_bytes(int d, int nw) {
    return (size_t)2 * kMfmaMaxQ * (d + 8) * sizeof(uint16_t) + (size_t)nw * 4096;
}

hipError_t prepare_mfma_filter() {
    hipError_t err = hipSuccess;
#define RT_PREP(NCK, NW, KPF)                                                                                 \
    if (err == hipSuccess)                                                                                    \
        err = hipFuncSetAttribute(reinterpret_cast<const void *>(&mfma_bound_kernel<NCK, NW, KPF>),           \
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)bound_lds_bytes(NCK * 64, NW));
    RT_BOUND_DEPTHS(RT_PREP)
#undef RT_PREP
    return err;
}

hipError_t launch_mfma_bound(const uint16_t *corpus16, int64_t n, int d, const float *queries, int q,
                             const float *rnorm, const float *rerr, float *ubuf, int64_t uld, float *tlb, int64_t tld,
                             int num_cus, hipStream_t stream) {
    const int64_t tiles = (n + 31) / 32;
    float cr, cx, delta;
    filter_bound_constants_batched(d, &cr, &cx, &delta);
#define RT_LAUNCH(NCK, NW, KPF)                                                                                 \
    if (d == NCK * 64) {                                                                                        \
        const int64_t tpw = (tiles + (int64_t)num_cus * NW - 1) / ((int64_t)num_cus * NW);                      \
        const int64_t blocks = (tiles + tpw * NW - 1) / (tpw * NW);                                             \
        hipLaunchKernelGGL((mfma_bound_kernel<NCK, NW, KPF>), dim3((unsigned)blocks), dim3(64 * NW),            \
                           bound_lds_bytes(d, NW), stream, corpus16, n, queries, q, rnorm, rerr, cr, cx, delta,  \
                           ubuf, uld, tlb, tld, tpw);                                                           \
        return hipGetLastError();                                                                               \
    }
    RT_BOUND_DEPTHS(RT_LAUNCH)
#undef RT_LAUNCH
    return hipErrorInvalidValue;
}

}  // namespace rt
