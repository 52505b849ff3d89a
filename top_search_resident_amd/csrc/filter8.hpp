// filter8.hpp -- the first pass of the filtered search over an fp8 copy of the
// corpus (gfx950; one query per segment).
//
// Same method as the bf16 first pass (filter_topk.hpp): the pages' plan of
// reduced-precision storage with an exact re-rank ("CUDA Programming Model
// Series 9: Efficient TopK", section 4.3), with certified bounds so that the
// answer stays the plain scan's.  Here each row x is stored as e4m3 codes of
// x / s with a power-of-two scale s per row (max |x / s| <= 224, inside the
// finite range of both e4m3 variants), so a row takes D bytes: a quarter of the
// fp32 row.  Per row the pass computes
//   a = s * (sum_j dec(c_j) q_j)    (fp32 FMA chain + group_sum; times s, exact)
// where x~_j = s dec(c_j) is the stored value, and the bound
//   |a - s_plain| <= |q| (cr |x - x~| + cx |x|) + delta max(|q|, 1) max(s, 1),
// cr = (1 + gamma_D)(1 + 2^-10), cx = 2 gamma_D (1 + 2^-10), gamma_D =
// D u / (1 - D u), u = 2^-24: Cauchy-Schwarz on the rounding error vector
// (|x - x~| computed per row from the stored codes, rounded up), gamma_D for
// the fp32 sum of a over sum |x~_j q_j| <= (|x| + |x - x~|) |q| and gamma_D for
// the plain scan's sum; delta = 4 D 2^-126 covers underflow of products and
// partial sums (scaled by s in a).  The row's part of the bound, c = cr |x - x~|
// + cx |x|, is computed with the copy and stored beside s (one float2 per row),
// so a row costs D + 8 bytes to read and e = |q| c + delta max(|q|, 1) max(s, 1)
// (the fp32 roundings of c and e are far inside the 2^-10 slack of cr and cx).
// The upper bound a + e is stored and the lower bound a - e ranked; the tree's
// root writes the k-th lower bound, and the bf16 path's second pass
// (gemv_filtered_kernel) re-scores the rows whose upper bound reaches it.  The
// error norm of an e4m3 row is ~0.027 |x| for Gaussian rows (bf16: ~0.0017
// |x|), so many more rows reach the threshold; the pass pays only where the
// corpus is large.
#pragma once
#include "filter_topk.hpp"

namespace rt {

// Extra per-row data of the fp8 first pass.
struct Fp8Rows {
    const uint8_t *codes;  // n x d e4m3 codes, row-major
    const float2 *meta;    // per row {s (a power of two), c = cr |x - x~| + cx |x|}
    float delta;           // bound constant
};

__device__ __forceinline__ float fp8_block_dot(const uint4 &v, const float4 (&q)[4], float a) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
        const float4 qq = q[i];
        a = fmaf(lo[0], qq.x, a);
        a = fmaf(lo[1], qq.y, a);
        a = fmaf(hi[0], qq.z, a);
        a = fmaf(hi[1], qq.w, a);
    }
    return a;
}

// Lane-group layout as gemv_bound_kernel, over 16-byte blocks of 16 codes (d16 =
// d / 16 blocks per row, exactly G L: the launcher checks it, so no block is
// padded): lane g of a group of G = 2^LG lanes owns blocks g, g + G, ... (L
// loads); loads run P steps ahead.
// COS: cosine bounds from fa.crn (the rows' L2 norms, 4 more bytes per row).
template <int LG, int L, int R, int P, bool COS>
__global__ __launch_bounds__(64 * gemv_waves(64 * R)) void gemv_bound8_kernel(
    Fp8Rows fr, int64_t n, int d, const float *__restrict__ queries, int64_t rows_per_wave, TreeArgs ta,
    FilterArgs fa) {
    constexpr int G = 1 << LG;
    constexpr int RPS = 64 >> LG;
    constexpr int U = RowUnroll<L>::value;
    constexpr int STEP = RPS * U;
    constexpr int W = gemv_waves(64 * R);
    static_assert(P > 0, "loads always run ahead");
    __shared__ uint64_t stage[W][128];
    __shared__ uint64_t sm[kTreeEntries];
    __shared__ MergeScratch ms;
    // 16-bit upper bounds are gathered per wave in LDS and written kBurst rows
    // at a time (the wave's whole range at 1M rows): writes in bursts between
    // long stretches of reads cost the read stream less than one 2-byte store
    // per row spread over it (1M x 1024, whole search at K = 8 / 100, device
    // p50 on MI355X: 192.4 / 210.5 against 195.2 / 213.4 us).
    constexpr int kBurst = 2048;
    __shared__ uint16_t bst[W][kBurst];

    const int seg = blockIdx.y;
    const int lane = lane_id();
    const int wv = wave_in_group();
    const int64_t wave = (int64_t)blockIdx.x * W + wv;
    const int g = lane & (G - 1);
    const int h = lane >> LG;
    const int d16 = d >> 4;
    const float *qrow = queries + (int64_t)seg * d;
    uint64_t *const my_stage = stage[wv];
    float *const ub = fa.ubuf + (int64_t)seg * fa.uld;

    WaveSelector<R> sel;
    sel.init(ta.k);
    const float qnorm = wave_l2_norm(qrow, d);
    const float dl = fr.delta * fmaxf(qnorm, 1.f);

    // The sixteen query values of each of this lane's blocks.
    float4 qv[L][4];
    int colc[L];
#pragma unroll
    for (int j = 0; j < L; ++j) {
        colc[j] = j * G + g;
        const float4 *q4 = reinterpret_cast<const float4 *>(qrow) + 4 * colc[j];
#pragma unroll
        for (int i = 0; i < 4; ++i) qv[j][i] = q4[i];
    }

    const int64_t r_begin = wave * rows_per_wave;
    const int64_t r_end = (r_begin + rows_per_wave < n) ? r_begin + rows_per_wave : n;
    if (r_begin < r_end) {
        uint16_t *const my_bst = bst[wv];
        int64_t blk = r_begin;
        auto flush = [&](int64_t b0, int64_t b1) {
            wave_lds_sync();
            uint16_t *const dst = fa.ub16_out + (int64_t)seg * fa.uld;
            for (int64_t r = b0 + lane; r < b1; r += 64) dst[r] = my_bst[r - b0];
            wave_lds_sync();
        };
        const uint4 *__restrict__ c8 = reinterpret_cast<const uint4 *>(fr.codes);
        const int64_t last = r_end - 1;
        uint4 x[P][U][L];
        float2 mt[P][U];
        float cn[P][U];
        auto load_step = [&](int s, int64_t r0) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                int64_t row = r0 + u * RPS + h;
                row = row < last ? row : last;
                const uint4 *p = c8 + row * d16;
#pragma unroll
                for (int j = 0; j < L; ++j) x[s][u][j] = load_nt(p + colc[j]);
                mt[s][u] = fr.meta[row];
                if constexpr (COS) cn[s][u] = fa.crn[row];
            }
        };
        auto consume = [&](int s, int64_t rs0) {
            float lo[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float a = 0.f;
#pragma unroll
                for (int j = 0; j < L; ++j) a = fp8_block_dot(x[s][u][j], qv[j], a);
                const float sc = mt[s][u].x;
                a = group_sum(a, LG) * sc;
                const float e = fmaf(qnorm, mt[s][u].y, dl * fmaxf(sc, 1.f));
                const int64_t row = rs0 + u * RPS + h;
                // false for an overflowed or NaN sum or bound: the row is kept
                const bool known = fabsf(a) <= __FLT_MAX__ && e <= __FLT_MAX__;
                float hi = known ? a + e : __builtin_huge_valf();
                float lw = known ? a - e : -__builtin_huge_valf();
                if constexpr (COS) cosine_bounds(known, a, e, qnorm, cn[s][u], hi, lw);
                if (g == 0 && row < r_end) {
                    if (fa.ub16_out)  // uniform
                        my_bst[row - blk] = bf16_round_up_bits(hi);
                    else
                        ub[row] = hi;
                }
                lo[u] = lw;
            }
            load_step(s, rs0 + P * STEP);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t row = rs0 + u * RPS + h;
                const bool valid = (g == 0) && (row < r_end);
                const uint64_t rank = make_rank(order_key_f32(lo[u]), (uint32_t)row);
                sel.offer(my_stage, rank, valid && rank > sel.thr);
            }
        };
#pragma unroll
        for (int s = 0; s < P; ++s) {
            load_step(s, r_begin + s * STEP);
            __builtin_amdgcn_sched_barrier(0);
        }
        const bool bursts = fa.ub16_out != nullptr;
        for (int64_t r0 = r_begin; r0 < r_end; r0 += P * STEP) {
            if (bursts && r0 - blk >= kBurst) {
                flush(blk, r0);
                blk = r0;
            }
#pragma unroll
            for (int s = 0; s < P; ++s) consume(s, r0 + s * STEP);
        }
        if (bursts) flush(blk, r_end);
    }
    sel.finish(my_stage);
    finish_workgroup<R, W * 64>(sel, sm, &ms, ta, seg);
}

}  // namespace rt
