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
//     per (query, row) as a 16-bit value rounded up (still an upper bound),
//     and per query the largest lower bound a - e of every 32-row tile;
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
#include "lds_dma.hpp"

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
                                                            float delta, uint16_t *__restrict__ ub16,
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
        // Bounds of the tile's rows for query m: upper bounds stored as 16-bit
        // values rounded up, tile-major (tile t's block of 32 q entries at
        // 32 t q, query m's rows at 32 m in it: the four stores of a tile fill
        // its 64 q bytes, 16 contiguous bytes per query and instruction), the
        // tile's largest lower bound kept.
        float mx = -__builtin_huge_valf();
        uint16_t *const ublk = ub16 + t * 32 * q + m * 32 + 4 * h;
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
                if (has_q)
                    *reinterpret_cast<uint2 *>(ublk + 8 * gg) =
                        make_uint2((uint32_t)bf16_round_up_bits(ubv[0]) | ((uint32_t)bf16_round_up_bits(ubv[1]) << 16),
                                   (uint32_t)bf16_round_up_bits(ubv[2]) | ((uint32_t)bf16_round_up_bits(ubv[3]) << 16));
                mx = fmaxf(mx, fmaxf(fmaxf(lbv[0], lbv[1]), fmaxf(lbv[2], lbv[3])));
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if (r + c < n) {
                        if (has_q) ublk[8 * gg + c] = bf16_round_up_bits(ubv[c]);
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

// Pass 1 through direct loads, for d = 64 NCK with NCK in {4, 6, 8, 12}: one
// wave per SIMD, the query's bf16 hi and lo parts in registers (d / 2
// registers per lane: 384 at d = 768), the corpus streamed into a ring of NR
// 4 KB chunk slots in the wave's own LDS (32 rows x 128 bytes, loaded as 8 rows
// x 128 contiguous bytes per instruction with the non-temporal hint, unit u of
// row r at position u ^ f(r)), and each tile's row norms and error norms
// loaded the same way into one of two small LDS slots (so no ordinary global
// load is ever outstanding next to the ring: the compiler would drain the
// ring to wait for it).  The MFMA layout is the one above (lane (m, h) takes
// unit 2 s + h of row m for k-step s; hi and lo parts: two MFMAs per k-step).
// The upper bounds are written as 16-bit values rounded toward +inf (the top
// half of an fp32 word, incremented when a positive value loses bits), which
// halves the bytes written -- in this streaming pass every byte written costs
// more than a byte read (measured on MI355X: 64 MB of scattered writes next to
// a full-rate read stream cost ~70 us, 16 MB ~30 us) -- at the price of a
// slightly wider candidate band in pass 2 (2^-8 relative).  They are laid out
// tile-major: tile t's bounds are one block of 32 q entries at ub16 + 32 t q,
// query j's 32 rows at offset 32 j, transposed through LDS so that each store
// instruction writes 1 KB of contiguous lines (query-major rows, i.e. 64-byte
// runs 1 MB apart, took 185.5 against 175.5 us at 32 x 500k x 768, measured
// on MI355X; pass 2's half-line reads cost it ~2 us of that back).  A ragged
// last tile is loaded from row n - 32; only its rows from 32 t on are written.

template <int NCK>
struct BoundRing {
    static constexpr int value = (NCK % 8 == 0) ? 8 : (NCK % 6 == 0 ? 6 : 4);
};

template <int NCK>
struct BoundDma {
    // At d = 768 the lo parts stay in LDS (with both parts in registers the
    // kernel needs more than 512 of them), which leaves room for 6 chunk slots.
    static constexpr bool kLoInLds = NCK > 8;
    // chunk slots (<= NCK: the prologue fills them from the first tile); NR - 1
    // chunks are loading while one is read
    static constexpr int kRing = kLoInLds ? 6 : (NCK < 8 ? NCK : 8);
    static constexpr int kLoStride = NCK * 128 + 16;  // bytes per query row of lo parts (padded)
    static constexpr int kWaveLds = kRing * 4096 + 2048 + 512;  // ring, bound stage, two norm slots
    static constexpr int kLoLds = kLoInLds ? 32 * kLoStride : 0;
    static constexpr int kLds = kLoLds + 4 * kWaveLds;
};

template <int NCK>
__global__ __launch_bounds__(256, 1) void mfma_bound_dma_kernel(const uint16_t *__restrict__ corpus16, int64_t n,
                                                                const float *__restrict__ queries, int q,
                                                                const float *__restrict__ rnorm,
                                                                const float *__restrict__ rerr, float cr, float cx,
                                                                float delta, uint16_t *__restrict__ ub16,
                                                                float *__restrict__ tlb, int64_t tld) {
    using L = BoundDma<NCK>;
    constexpr int d = NCK * 64;
    constexpr int NR = L::kRing;
    static_assert(NR >= 4 && NR <= NCK, "ring");
    static_assert(L::kLds + 32 * 4 <= 160 * 1024, "LDS");
    // [lo parts of the query block, at d = 768] then per wave: NR chunk slots of
    // 4 KB, a 2 KB stage for the bounds, two 256-byte norm slots
    extern __shared__ __align__(16) char bound_lds[];
    const int lane = threadIdx.x & 63;
    const int wv = wave_in_group();
    const int m = lane & 31;
    const int h = lane >> 5;
    const int64_t wave = (int64_t)blockIdx.x * 4 + wv;
    const int64_t tiles = (n + 31) / 32;
    // The tiles are split evenly over all waves (runs of floor or ceil of
    // tiles / waves): with a fixed run length, at 500k rows 1024 waves of 16
    // tiles left 11 of the 256 CUs idle (whole batch 208.5 against 202.9 us at
    // K = 100, measured on MI355X).
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    const int64_t t_begin = wave * tiles / nwaves;
    const int64_t t_end = (wave + 1) * tiles / nwaves;
    char *const lo_lds = bound_lds;
    char *const wave_lds = bound_lds + L::kLoLds;
    __shared__ float qn_s[32];

    // The fp32 query block goes through LDS first (coalesced loads by the whole
    // workgroup into the per-wave space, not yet in use); each wave computes
    // the L2 norms of eight queries from it (as the other bound kernel does),
    // and each lane builds query m's hi and lo parts for k-step s of chunk c
    // (columns 64 c + 8 (2 s + h) .. + 7).
    static_assert(32 * d * 4 <= 4 * L::kWaveLds, "query block fits the per-wave space");
    {
        float4 *qs4 = reinterpret_cast<float4 *>(wave_lds);
        for (int i = threadIdx.x; i < 32 * d / 4; i += 256) {
            const int r = i / (d / 4);
            qs4[i] = (r < q) ? reinterpret_cast<const float4 *>(queries)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    __syncthreads();
    for (int j = wv; j < 32; j += 4) {
        const float v = wave_l2_norm(reinterpret_cast<const float *>(wave_lds) + j * d, d);
        if (lane == 0) qn_s[j] = v;
    }
    uint4 qh[NCK][4];
    uint4 ql[L::kLoInLds ? 1 : NCK][4];
    {
        const float *qrow = reinterpret_cast<const float *>(wave_lds) + m * d + 8 * h;
#pragma unroll
        for (int c = 0; c < NCK; ++c)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float4 v0 = *reinterpret_cast<const float4 *>(qrow + 64 * c + 16 * s);
                const float4 v1 = *reinterpret_cast<const float4 *>(qrow + 64 * c + 16 * s + 4);
                const float x[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
                uint32_t hw[4], lw[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x0 = x[2 * e], x1 = x[2 * e + 1];
                    const uint32_t h0 = bf16_bits_rne(x0), h1 = bf16_bits_rne(x1);
                    hw[e] = h0 | (h1 << 16);
                    lw[e] = bf16_bits_rne(x0 - __uint_as_float(h0 << 16)) |
                            (bf16_bits_rne(x1 - __uint_as_float(h1 << 16)) << 16);
                }
                qh[c][s] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
                if constexpr (L::kLoInLds)
                    *reinterpret_cast<uint4 *>(lo_lds + m * L::kLoStride + (64 * c + 8 * (2 * s + h)) * 2) =
                        make_uint4(lw[0], lw[1], lw[2], lw[3]);
                else
                    ql[c][s] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
                // one k-step at a time: hoisting every LDS read of the block
                // ahead of the conversions would need ~d more registers
                __builtin_amdgcn_sched_barrier(0);
            }
    }
    __syncthreads();  // every wave has its query parts before any ring slot is loaded
    if (t_begin >= t_end) return;  // no barrier follows
    const float qn = qn_s[m];
    const float er = cr * qn;
    const float ex = cx * qn;
    const float dl = delta * fmaxf(qn, 1.f);
    const bool has_q = m < q;

    char *const ring = wave_lds + wv * L::kWaveLds;
    char *const stage = ring + NR * 4096;
    char *const norms = stage + 2048;  // two 256-byte slots: [rnorm 32 floats][rerr 32 floats]
    const uint32_t ring_lds = lds_addr(ring);
    const uint32_t norms_lds = lds_addr(norms);
    const char *const lo_row = lo_lds + m * L::kLoStride + 16 * h;
    int voff[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int r = 8 * p + (lane >> 3);
        const int u = (lane & 7) ^ dma_swizzle(r);
        voff[p] = (r * d + u * 8) * 2;
    }
    int roff[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) roff[s] = m * 128 + (((2 * s + h) ^ dma_swizzle(m)) << 4);
    auto load_row0 = [&](int64_t t) -> int64_t {
        const int64_t r = t * 32;
        return (r + 32 > n) ? n - 32 : r;
    };
    auto issue = [&](int64_t lr0, int c, int slot) {
        const char *base = reinterpret_cast<const char *>(corpus16 + lr0 * d + c * 64);
#pragma unroll
        for (int p = 0; p < 4; ++p) dma16_nt(base, voff[p], ring_lds + slot * 4096 + p * 1024);
    };
    // rows lr0 .. lr0 + 31: lanes 0..7 their norms, lanes 8..15 their error
    // norms, 256 bytes (the other lanes are masked off: one load instruction)
    auto issue_norms = [&](int64_t lr0, int par) {
        if (lane < 16) {
            const float *src = (lane < 8) ? rnorm + lr0 + 4 * lane : rerr + lr0 + 4 * (lane - 8);
            dma16_nt_addr(src, norms_lds + par * 256);
        }
    };
    // Chunks are numbered across the wave's tiles; chunk g lives in slot g % NR
    // (wave-uniform counters, not compile-time: NR need not divide NCK).  Once
    // the operands of chunk g have been read, its slot is refilled with chunk
    // g + NR, so NR - 1 chunks are loading while chunk g + 1 is waited for.
    const int64_t lr_first = load_row0(t_begin);
    issue_norms(lr_first, 0);
#pragma unroll
    for (int c = 0; c < NR; ++c) issue(lr_first, c, c);
    int slot_cur = 0;  // slot of chunk g
    uint4 a[2][4];
    uint4 lo[2][4];  // lo parts of the chunk's query operands when they are kept in LDS
    wait_vmcnt<4 * (NR - 1)>();  // the norms and chunk 0 have landed
#pragma unroll
    for (int s = 0; s < 4; ++s) a[0][s] = *reinterpret_cast<const uint4 *>(ring + roff[s]);
    if constexpr (L::kLoInLds) {
#pragma unroll
        for (int s = 0; s < 4; ++s) lo[0][s] = *reinterpret_cast<const uint4 *>(lo_row + 32 * s);
    }
    // The bounds and tile maxima of up to kHeld full tiles are held back in
    // registers (wave-uniform count) and written together with the next
    // tile's: 16 tiles' bounds as one 32 KB run, 16 maxima per query as one
    // 64-byte run.  Writes issued in bursts between long stretches of reads
    // cost the read stream less than the same writes spread over it (32 x 500k
    // x 768, whole batch at K = 100, measured on MI355X: one tile at a time
    // 224.7 us, 2 tiles 219.5, 4 217.2, 8 212.0, 16 209.1, and 16 with the
    // maxima held too 209.7 against 212.7).
    constexpr int kHeld = 15;
    uint32_t held[kHeld][4][2] = {};
    float heldmx[kHeld] = {};
    int held_n = 0;
    for (int64_t t = t_begin; t < t_end; ++t) {
        const int64_t lr = load_row0(t);
        const int64_t lr_next = (t + 1 < t_end) ? load_row0(t + 1) : lr;  // past the last tile: reload, unused
        const int par = (int)((t - t_begin) & 1);
        floatx16 acc;
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
        for (int c = 0; c < NCK; ++c) {
            const int slot_next = (slot_cur + 1 == NR) ? 0 : slot_cur + 1;
            // this chunk's corpus operands are in registers (the asm waits for
            // their LDS reads); refill its slot with chunk c + NR (the next
            // tile's chunk c + NR - NCK past the end, with that tile's norms)
            asm volatile("" ::"v"(a[c & 1][0].x), "v"(a[c & 1][1].x), "v"(a[c & 1][2].x), "v"(a[c & 1][3].x));
            __builtin_amdgcn_sched_barrier(0);
            {
                const int cn = c + NR;  // a constant once the loop is unrolled
                if (cn < NCK) {
                    issue(lr, cn, slot_cur);
                } else {
                    if (cn == NCK) issue_norms(lr_next, par ^ 1);
                    issue(lr_next, cn - NCK, slot_cur);
                }
            }
            // chunk c + 1 must have landed: the loads after it are chunks c + 2 .. c + NR
            // (and perhaps the next tile's norms)
            wait_vmcnt<4 * (NR - 1)>();
            __builtin_amdgcn_sched_barrier(0);
            {
                const char *src = ring + slot_next * 4096;
#pragma unroll
                for (int s = 0; s < 4; ++s) a[(c + 1) & 1][s] = *reinterpret_cast<const uint4 *>(src + roff[s]);
            }
            if constexpr (L::kLoInLds) {
                const int cq = (c + 1 < NCK) ? c + 1 : 0;  // the next tile starts again at chunk 0
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    lo[(c + 1) & 1][s] = *reinterpret_cast<const uint4 *>(lo_row + (64 * cq + 16 * s) * 2);
            }
            slot_cur = slot_next;
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 av = __builtin_bit_cast(bf16x8, a[c & 1][s]);
                const uint4 qlo = L::kLoInLds ? lo[c & 1][s] : ql[L::kLoInLds ? 0 : c][s];
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8, qh[c][s]), acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8, qlo), acc, 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // Bounds of rows lr + 8 g + 4 h + c' for query m (register 4 g + c').
        const char *nslot = norms + par * 256;
        const int64_t row0 = t * 32;
        float mx = -__builtin_huge_valf();
        uint32_t packed[4][2];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 rn = *reinterpret_cast<const float4 *>(nslot + (8 * g + 4 * h) * 4);
            const float4 re = *reinterpret_cast<const float4 *>(nslot + 128 + (8 * g + 4 * h) * 4);
            uint16_t u16[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float av = acc[4 * g + c];
                const float rv = comp4(rn, c);
                const float e = fmaf(er, comp4(re, c), fmaf(ex, rv, dl * fmaxf(rv, 1.f)));
                // false for an overflowed or NaN sum or bound: the row is kept
                const bool known = fabsf(av) <= __FLT_MAX__ && e <= __FLT_MAX__;
                const float ubv = known ? av + e : __builtin_huge_valf();
                const float lbv = known ? av - e : -__builtin_huge_valf();
                u16[c] = bf16_round_up_bits(ubv);
                if (lr + 8 * g + 4 * h + c >= row0) mx = fmaxf(mx, lbv);
            }
            packed[g][0] = (uint32_t)u16[0] | ((uint32_t)u16[1] << 16);
            packed[g][1] = (uint32_t)u16[2] | ((uint32_t)u16[3] << 16);
        }
        const float mx_all = fmaxf(mx, __uint_as_float(xor_u32<32>(__float_as_uint(mx))));
        auto store_tile = [&](const uint32_t (&pk)[4][2], int64_t r0) {
            // stage [query][32 rows] x 2 bytes, then 4 lanes x 16 bytes per query run
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<uint2 *>(stage + m * 64 + (8 * g + 4 * h) * 2) = make_uint2(pk[g][0], pk[g][1]);
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int jj = 16 * k + (lane >> 2);
                const int su = lane & 3;
                const uint4 v = *reinterpret_cast<const uint4 *>(stage + jj * 64 + su * 16);
                if (jj < q) {
                    const u32x4_t w = {v.x, v.y, v.z, v.w};
                    __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t *>(ub16 + r0 * q + jj * 32 + 8 * su));
                }
            }
        };
        if (lr == row0) {
            if (held_n < kHeld && t + 1 < t_end && load_row0(t + 1) == row0 + 32) {
#pragma unroll
                for (int i = 0; i < kHeld; ++i)
                    if (i == held_n) {
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            held[i][g][0] = packed[g][0];
                            held[i][g][1] = packed[g][1];
                        }
                        heldmx[i] = mx_all;
                    }
                ++held_n;
                continue;
            }
#pragma unroll
            for (int i = 0; i < kHeld; ++i)
                if (i < held_n) {
                    store_tile(held[i], row0 - 32 * (held_n - i));
                    if (h == 0 && has_q) tlb[(int64_t)m * tld + t - (held_n - i)] = heldmx[i];
                }
            held_n = 0;
            store_tile(packed, row0);
        } else if (has_q) {  // the ragged last tile, loaded from n - 32: rows from row0 on
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int64_t r = lr + 8 * g + 4 * h + c;
                    if (r >= row0) ub16[row0 * q + m * 32 + (r - row0)] = (uint16_t)(packed[g][c >> 1] >> (16 * (c & 1)));
                }
        }
        if (h == 0 && has_q) tlb[(int64_t)m * tld + t] = mx_all;
    }
    wait_vmcnt<0>();  // no direct load may still be writing LDS when the wave ends
}

#define RT_BOUND_DMA(X) X(4) X(6) X(8) X(12)

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
#define RT_PREP_DMA(NCK)                                                                                  \
    if (err == hipSuccess)                                                                                \
        err = hipFuncSetAttribute(reinterpret_cast<const void *>(&mfma_bound_dma_kernel<NCK>),            \
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)(size_t)BoundDma<NCK>::kLds);
    RT_BOUND_DMA(RT_PREP_DMA)
#undef RT_PREP_DMA
    return err;
}

hipError_t launch_mfma_bound(const uint16_t *corpus16, int64_t n, int d, const float *queries, int q,
                             const float *rnorm, const float *rerr, float *ubuf, float *tlb, int64_t tld,
                             int num_cus, hipStream_t stream) {
    const int64_t tiles = (n + 31) / 32;
    float cr, cx, delta;
    filter_bound_constants_batched(d, &cr, &cx, &delta);
    if (n >= 32) {
        const int64_t blocks = ((tiles + 3) / 4 < num_cus) ? (tiles + 3) / 4 : num_cus;
#define RT_LAUNCH_DMA(NCK)                                                                                      \
        if (d == NCK * 64) {                                                                                    \
            hipLaunchKernelGGL((mfma_bound_dma_kernel<NCK>), dim3((unsigned)blocks), dim3(256),                 \
                               (size_t)BoundDma<NCK>::kLds, stream, corpus16, n, queries, q, rnorm, rerr, cr, cx,  \
                               delta, reinterpret_cast<uint16_t *>(ubuf), tlb, tld);                            \
            return hipGetLastError();                                                                           \
        }
        RT_BOUND_DMA(RT_LAUNCH_DMA)
#undef RT_LAUNCH_DMA
    }
#define RT_LAUNCH(NCK, NW, KPF)                                                                                 \
    if (d == NCK * 64) {                                                                                        \
        const int64_t tpw = (tiles + (int64_t)num_cus * NW - 1) / ((int64_t)num_cus * NW);                      \
        const int64_t blocks = (tiles + tpw * NW - 1) / (tpw * NW);                                             \
        hipLaunchKernelGGL((mfma_bound_kernel<NCK, NW, KPF>), dim3((unsigned)blocks), dim3(64 * NW),            \
                           bound_lds_bytes(d, NW), stream, corpus16, n, queries, q, rnorm, rerr, cr, cx, delta,  \
                           reinterpret_cast<uint16_t *>(ubuf), tlb, tld, tpw);                                  \
        return hipGetLastError();                                                                               \
    }
    RT_BOUND_DEPTHS(RT_LAUNCH)
#undef RT_LAUNCH
    return hipErrorInvalidValue;
}

}  // namespace rt
