// filter_topk.hpp -- exact inner-product top-K that reads a bf16 copy of the
// corpus first and the fp32 rows only where they can matter (gfx950).
//
// "GPU-Resident Top-K for Agentic RAG" (A. Banerjee) scores every row in fp32
// (section 4, Step 2); the scan is bound by reading N x D x 4 bytes.  With a
// bf16 copy of the corpus resident as well, a first pass reads half the bytes:
// for row i it computes a_i = sum_j bf16(x_ij) q_j in fp32 and a bound e_i with
// |a_i - s_i| <= e_i, where s_i is the fp32 score the plain path computes.
// The bound follows from the rounding of x to bf16 (8 significant bits, so
// round-to-nearest-even is off by at most 2^-8 relative) and from the fp32
// summation error of both sums (gamma_D = D u / (1 - D u), u = 2^-24, times
// the sum of |terms|), with sum_j |x_ij q_j| <= |x_i| |q| (Cauchy-Schwarz):
//     e_i = |x_i| |q| (2^-8 + gamma_D (2 + 2^-8)), rounded up (host: cb),
// plus 4 D 2^-126 max(|q|, 1), which covers the absolute rounding of values
// below 2^-126 and of products and sums that underflow (flushed or not) in
// both sums.  A bf16 sum or bound that is not finite bounds nothing: that row
// gets the bounds -inf and +inf (always re-scored, never sets T).  The first
// pass finds T, the k-th largest lower bound a_i - e_i (k rows have s_i >= T),
// and stores every upper bound a_i + e_i.  Any row with a_i + e_i < T has
// s_i < T <= the k-th largest s, so the top-k by s lies among the rows with
// a_i + e_i >= T: the second pass re-scores exactly those rows in fp32 with
// the plain path's arithmetic (lane_chain + group_sum) and selects among them.
// The answer is the plain path's answer, bit for bit.  For Gaussian unit rows
// at 1M x 1024 and k = 100 the band [T - 2 e, T] holds a few hundred rows, so
// the second pass reads ~4 MB of bounds and a few hundred fp32 rows.
#pragma once
#include <type_traits>

#include "stream_topk.hpp"

namespace rt {

// Extra arguments of the two passes.
struct FilterArgs {
    float cb;        // bound factor: e_i = cb |q| |x_i| + delta
    float delta;     // absolute slack for underflow, times max(|q|, 1)
    float *ubuf;     // [segments][uld] upper bounds a_i + e_i (pass 1 writes, pass 2 reads)
    int64_t uld;
    float *thr;      // [segments] T, the k-th largest lower bound (written by pass 1's tree)
    const float *crn;  // cosine metric: the rows' L2 norms (null for the inner product)
    const uint16_t *ub16;  // pass 2: 16-bit upper bounds (top halves of fp32, rounded up) instead of ubuf
    uint16_t *ub16_out;    // pass 1: write the upper bounds here as 16-bit values instead of to ubuf
    int ub_tq;             // nonzero: ub16 is tile-major, 32-row tiles of ub_tq queries x 32 rows each
    uint64_t *cand;        // pass 2, collect mode: the wave over rows [r0, r1) writes its
                           // candidates' ranks to cand[seg * cand_ld + r0 ..] (cand_ld >= n)
    int64_t cand_ld;
    uint32_t *cand_cnt;    // and their number to cand_cnt[seg * cnt_ld + wave], every wave
    int64_t cnt_ld;
};

// The top half of an fp32 value's bits, rounded toward +inf (bf16 rounded
// up): positive and inexact, the next bf16 up (values above the largest bf16
// go to +inf); zero, negative or exact, dropping the low bits moves toward
// zero or changes nothing.  Either way the 16-bit value, widened, is >= x, so
// an upper bound stays an upper bound.
__device__ __forceinline__ uint16_t bf16_round_up_bits(float x) {
    const uint32_t b = __float_as_uint(x);
    const uint32_t hi = b >> 16;
    return (uint16_t)((!(b >> 31) && (b & 0xffffu)) ? hi + 1u : hi);
}

// bf16 -> fp32 of the two halves of a 32-bit word.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Pass 1.  Lane-group layout as gemv_topk_kernel, over 16-byte blocks of 8 bf16
// (d8 = d / 8 blocks per row): lane g of a group of G = 2^LG lanes owns blocks
// g, g + G, ... (L loads).  Loads always run ahead (P = 2 or 4 steps): a bf16
// step carries half the bytes of an fp32 one, and with loads at use the pass
// reached only 4.7 TB/s at 1M x 1024 (432 us; 326 us with P = 2, 320 us with
// P = 4, measured on MI355X).  Per row: a (fp32 FMA chain per lane, group_sum), the
// bound e, the upper bound written to ubuf (as a 16-bit value rounded up,
// bf16_round_up_bits, when fa.ub16_out is set), the lower bound ranked by the
// wave selectors; the merge tree's root writes the k-th lower bound to thr[seg].
template <int LG, int L, int R, int P, bool COS>
__global__ __launch_bounds__(64 * gemv_waves(64 * R)) void gemv_bound_kernel(
    const uint16_t *__restrict__ corpus16, int64_t n, int d, const float *__restrict__ queries,
    const float *__restrict__ rnorm, int64_t rows_per_wave, TreeArgs ta, FilterArgs fa) {
    constexpr int G = 1 << LG;
    constexpr int RPS = 64 >> LG;
    constexpr int U = RowUnroll<L>::value;
    constexpr int STEP = RPS * U;
    constexpr int SLOTS = P > 0 ? P : 1;
    constexpr int W = gemv_waves(64 * R);
    __shared__ uint64_t stage[W][128];
    __shared__ uint64_t sm[kTreeEntries];
    __shared__ MergeScratch ms;

    const int seg = blockIdx.y;
    const int lane = lane_id();
    const int wv = wave_in_group();
    const int64_t wave = (int64_t)blockIdx.x * W + wv;
    const int g = lane & (G - 1);
    const int h = lane >> LG;
    const int d8 = d >> 3;
    const float *qrow = queries + (int64_t)seg * d;
    uint64_t *const my_stage = stage[wv];
    float *const ub = fa.ubuf + (int64_t)seg * fa.uld;

    WaveSelector<R> sel;
    sel.init(ta.k);
    const float qnorm = wave_l2_norm(qrow, d);
    const float eq = fa.cb * qnorm;
    const float dl = fa.delta * fmaxf(qnorm, 1.f);

    // The eight query values of each of this lane's blocks; blocks past the row
    // end load the last block and are and-ed with a zero mask.
    float4 qa[L], qb[L];
    int colc[L];
    uint32_t cmask[L];
#pragma unroll
    for (int j = 0; j < L; ++j) {
        const int col = j * G + g;
        const bool in = col < d8;
        colc[j] = in ? col : d8 - 1;
        cmask[j] = in ? 0xffffffffu : 0u;
        const float4 *q4 = reinterpret_cast<const float4 *>(qrow) + 2 * colc[j];
        qa[j] = in ? q4[0] : make_float4(0.f, 0.f, 0.f, 0.f);
        qb[j] = in ? q4[1] : make_float4(0.f, 0.f, 0.f, 0.f);
    }

    const int64_t r_begin = wave * rows_per_wave;
    const int64_t r_end = (r_begin + rows_per_wave < n) ? r_begin + rows_per_wave : n;
    if (r_begin < r_end) {
        const uint4 *__restrict__ c16 = reinterpret_cast<const uint4 *>(corpus16);
        const int64_t last = r_end - 1;
        uint4 x[SLOTS][U][L];
        float rn[SLOTS][U];
        auto load_step = [&](int s, int64_t r0) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                int64_t row = r0 + u * RPS + h;
                row = row < last ? row : last;
                const uint4 *p = c16 + row * d8;
#pragma unroll
                for (int j = 0; j < L; ++j) x[s][u][j] = load_nt(p + colc[j]);
                rn[s][u] = rnorm[row];
            }
        };
        auto consume = [&](int s, int64_t rs) {
            float lo[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float a = 0.f;
#pragma unroll
                for (int j = 0; j < L; ++j) {
                    uint4 v = x[s][u][j];
                    v.x &= cmask[j];
                    v.y &= cmask[j];
                    v.z &= cmask[j];
                    v.w &= cmask[j];
                    a = fmaf(bf16_lo(v.x), qa[j].x, a);
                    a = fmaf(bf16_hi(v.x), qa[j].y, a);
                    a = fmaf(bf16_lo(v.y), qa[j].z, a);
                    a = fmaf(bf16_hi(v.y), qa[j].w, a);
                    a = fmaf(bf16_lo(v.z), qb[j].x, a);
                    a = fmaf(bf16_hi(v.z), qb[j].y, a);
                    a = fmaf(bf16_lo(v.w), qb[j].z, a);
                    a = fmaf(bf16_hi(v.w), qb[j].w, a);
                }
                a = group_sum(a, LG);
                const float e = fmaf(eq, rn[s][u], dl);
                const int64_t row = rs + u * RPS + h;
                // false for an overflowed or NaN sum or bound: the row is kept
                const bool known = fabsf(a) <= __FLT_MAX__ && e <= __FLT_MAX__;
                float hi = known ? a + e : __builtin_huge_valf();
                float lw = known ? a - e : -__builtin_huge_valf();
                if constexpr (COS) cosine_bounds(known, a, e, qnorm, rn[s][u], hi, lw);
                if (g == 0 && row < r_end) {
                    if (fa.ub16_out)  // uniform
                        fa.ub16_out[(int64_t)seg * fa.uld + row] = bf16_round_up_bits(hi);
                    else
                        ub[row] = hi;
                }
                lo[u] = lw;
            }
            if constexpr (P > 0) {
                load_step(s, rs + P * STEP);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t row = rs + u * RPS + h;
                const bool valid = (g == 0) && (row < r_end);
                const uint64_t rank = make_rank(order_key_f32(lo[u]), (uint32_t)row);
                sel.offer(my_stage, rank, valid && rank > sel.thr);
            }
        };
        if constexpr (P == 0) {
            for (int64_t r0 = r_begin; r0 < r_end; r0 += STEP) {
                load_step(0, r0);
                consume(0, r0);
            }
        } else {
#pragma unroll
            for (int s = 0; s < P; ++s) {
                load_step(s, r_begin + s * STEP);
                __builtin_amdgcn_sched_barrier(0);
            }
            for (int64_t r0 = r_begin; r0 < r_end; r0 += P * STEP) {
#pragma unroll
                for (int s = 0; s < P; ++s) consume(s, r0 + s * STEP);
            }
        }
    }
    sel.finish(my_stage);
    finish_workgroup<R, W * 64>(sel, sm, &ms, ta, seg);
}

// Pass 2.  A wave takes rows_per_wave rows in chunks of 512: every lane reads
// eight upper bounds (one per block of 64 rows, all loaded at once), and the
// rows reaching T are listed in row order in the wave's LDS list (ballot +
// mbcnt).  The wave then scores the list C * RPS rows at a time: the loads of C
// rows per lane group are issued together (a wave's few candidates are spread
// over its chunk, so taking them together saves a round trip to memory per
// candidate), then each row is reduced exactly as gemv_topk_kernel does
// (lane_chain + group_sum with the same shape) and offered to the selectors.
// Rows below T are never read.
template <int LG, int L, int R, bool COS>
__global__ __launch_bounds__(64 * gemv_waves(64 * R)) void gemv_filtered_kernel(
    const float *__restrict__ corpus, int64_t n, int d, const float *__restrict__ queries,
    int64_t rows_per_wave, TreeArgs ta, FilterArgs fa) {
    constexpr int G = 1 << LG;
    constexpr int RPS = 64 >> LG;
    constexpr int NB = 8;  // blocks of 64 bounds loaded at once
    constexpr int C = (16 / L) < 1 ? 1 : ((16 / L) > 4 ? 4 : 16 / L);  // rows per lane group in flight
    constexpr int W = gemv_waves(64 * R);
    __shared__ uint64_t stage[W][128];
    __shared__ uint64_t sm[kTreeEntries];
    __shared__ MergeScratch ms;
    __shared__ uint16_t list[W][NB * 64];  // per wave: the chunk's rows reaching T

    const int seg = blockIdx.y;
    const int lane = lane_id();
    const int wv = wave_in_group();
    const int64_t wave = (int64_t)blockIdx.x * W + wv;
    const int g = lane & (G - 1);
    const int h = lane >> LG;
    const int d4 = d >> 2;
    uint16_t *const my_list = list[wv];
    const float4 *__restrict__ q4 = reinterpret_cast<const float4 *>(queries + (int64_t)seg * d);
    const float4 *__restrict__ c4 = reinterpret_cast<const float4 *>(corpus);
    const float *__restrict__ ub = fa.ubuf + (int64_t)seg * fa.uld;
    const uint16_t *__restrict__ ub16 =
        fa.ub16 ? fa.ub16 + (fa.ub_tq ? (int64_t)seg * 32 : (int64_t)seg * fa.uld) : nullptr;
    const int64_t ub_tile = (int64_t)fa.ub_tq * 32;  // entries per tile when tile-major
    uint64_t *const my_stage = stage[wv];

    WaveSelector<R> sel;
    sel.init(ta.k);
    const float T = fa.thr[seg];
    float qnorm = 0.f;  // the cosine's query norm, computed as the plain scan does
    if constexpr (COS) qnorm = wave_l2_norm(queries + (int64_t)seg * d, d);

    float4 qv[L];
    int colc[L];
    uint32_t cmask[L];
#pragma unroll
    for (int j = 0; j < L; ++j) {
        const int col = j * G + g;
        colc[j] = (col < d4) ? col : d4 - 1;
        cmask[j] = (col < d4) ? 0xffffffffu : 0u;
        qv[j] = (col < d4) ? q4[col] : make_float4(0.f, 0.f, 0.f, 0.f);
    }

    const int64_t r_begin = wave * rows_per_wave;
    const int64_t r_end = (r_begin + rows_per_wave < n) ? r_begin + rows_per_wave : n;
    uint32_t ncand = 0;  // wave-uniform: collect mode's kept rows
    for (int64_t b0 = r_begin; b0 < r_end; b0 += (int64_t)NB * 64) {
        float uu[NB];
        if (ub16) {  // wave-uniform
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int64_t row0 = b0 + b * 64 + lane;
                const int64_t row = row0 < r_end ? row0 : r_end - 1;
                const int64_t at = ub_tile ? (row >> 5) * ub_tile + (row & 31) : row;
                uu[b] = __uint_as_float((uint32_t)ub16[at] << 16);
            }
        } else {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int64_t row = b0 + b * 64 + lane;
                uu[b] = ub[row < r_end ? row : r_end - 1];
            }
        }
        int count = 0;  // wave-uniform
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const bool hit = b0 + b * 64 + lane < r_end && uu[b] >= T;
            const uint64_t mb = __ballot(hit);
            if (hit) my_list[count + lanes_below(mb)] = (uint16_t)(b * 64 + lane);
            count += __popcll(mb);
        }
        wave_lds_sync();
        // NC batches from list entry t0: entry t0 + c RPS + h goes to group h in
        // batch c; slots past the end re-read entry t0 (in cache) and offer
        // nothing, so loads and uses stay unconditional
        auto score = [&](auto nc, int t0) {
            constexpr int NC = decltype(nc)::value;
            const int first = my_list[t0];
            int mine[NC];
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int t = t0 + c * RPS + h;
                mine[c] = t < count ? (int)my_list[t] : -1;
            }
            float4 x[NC][L];
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int64_t row = b0 + (mine[c] >= 0 ? mine[c] : first);
#pragma unroll
                for (int j = 0; j < L; ++j) x[c][j] = c4[row * d4 + colc[j]];
            }
            __builtin_amdgcn_sched_barrier(0);  // all NC rows' loads before any use
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int64_t row = b0 + (mine[c] >= 0 ? mine[c] : first);
                float s = group_sum(lane_chain<G, L>(x[c], qv, cmask), LG);
                if constexpr (COS) s = cosine_of(s, qnorm, fa.crn[row]);
                const bool valid = (g == 0) && (mine[c] >= 0);
                const uint64_t rank = make_rank(order_key_f32(s), (uint32_t)row);
                if (fa.cand) {  // uniform: collect mode, the rank goes to the wave's slice of the list
                    // Scores below T are beaten by the k rows that certify T
                    // (NaN stays: it fails every comparison).
                    const bool keep = valid && !(s < T);
                    const uint64_t mk = __ballot(keep);
                    // a row is kept at most once, so the slice ends by r_end <= n <= cand_ld
                    const int64_t pos = r_begin + ncand + lanes_below(mk);
                    if (keep && pos < fa.cand_ld) fa.cand[(int64_t)seg * fa.cand_ld + pos] = rank;
                    ncand += (uint32_t)__popcll(mk);
                } else {
                    sel.offer(my_stage, rank, valid && rank > sel.thr);
                }
            }
        };
        for (int t0 = 0; t0 < count; t0 += C * RPS) {
            // most waves of a tight bound hold one batch or none
            if (count - t0 <= RPS)
                score(std::integral_constant<int, 1>{}, t0);
            else
                score(std::integral_constant<int, C>{}, t0);
        }
        wave_lds_sync();  // the list is rewritten by the next chunk
    }
    if (fa.cand) {  // collect mode (uniform over the grid): candidate_select_kernel selects
        if (lane == 0) fa.cand_cnt[(int64_t)seg * fa.cnt_ld + wave] = ncand;
        return;
    }
    sel.finish(my_stage);
    finish_workgroup<R, W * 64>(sel, sm, &ms, ta, seg);
}

inline FilterArgs make_filter(const FilterLaunch &f) {
    FilterArgs fa;
    fa.cb = f.cb;
    fa.delta = f.delta;
    fa.ubuf = f.ubuf;
    fa.uld = f.uld;
    fa.thr = f.thr;
    fa.crn = f.crn;
    fa.ub16 = f.bounds16 ? reinterpret_cast<const uint16_t *>(f.ubuf) : f.ub16;
    fa.ub16_out = f.bounds16 ? reinterpret_cast<uint16_t *>(f.ubuf) : nullptr;
    fa.ub_tq = f.bounds16 ? 0 : f.ub_tq;
    fa.cand = f.cand;
    fa.cand_ld = f.cand_ld;
    fa.cand_cnt = f.cand_cnt;
    fa.cnt_ld = f.cnt_ld;
    return fa;
}

// Launchers for lists of 64*R entries (shapes as RT_GEMV_SHAPES; pass 1 over
// 8-element bf16 blocks, pass 2 over float4 columns).
// `ahead`: short row ranges per wave (two steps ahead), else four.
template <int R>
hipError_t launch_bound_r(int lg, int L, bool ahead, dim3 grid, hipStream_t s, const uint16_t *corpus16, int64_t n,
                          int d, const float *queries, const float *rnorm, int64_t per_wave, const TreeLaunch &t,
                          const FilterLaunch &f) {
    const TreeArgs ta = make_tree(t);
    const FilterArgs fa = make_filter(f);
    const dim3 block(64 * gemv_waves(64 * R));
#define RT_SHAPE(LGV, LV)                                                                                         \
    if (lg == LGV && L == LV) {                                                                                   \
        if (ahead && fa.crn)                                                                                      \
            hipLaunchKernelGGL((gemv_bound_kernel<LGV, LV, R, 2, true>), grid, block, 0, s, corpus16, n, d,       \
                               queries, rnorm, per_wave, ta, fa);                                                 \
        else if (ahead)                                                                                           \
            hipLaunchKernelGGL((gemv_bound_kernel<LGV, LV, R, 2, false>), grid, block, 0, s, corpus16, n, d,      \
                               queries, rnorm, per_wave, ta, fa);                                                 \
        else if (fa.crn)                                                                                          \
            hipLaunchKernelGGL((gemv_bound_kernel<LGV, LV, R, 4, true>), grid, block, 0, s, corpus16, n, d,       \
                               queries, rnorm, per_wave, ta, fa);                                                 \
        else                                                                                                      \
            hipLaunchKernelGGL((gemv_bound_kernel<LGV, LV, R, 4, false>), grid, block, 0, s, corpus16, n, d,      \
                               queries, rnorm, per_wave, ta, fa);                                                 \
        return hipGetLastError();                                                                                 \
    }
    RT_GEMV_SHAPES(RT_SHAPE)
#undef RT_SHAPE
    return hipErrorInvalidValue;
}

template <int R>
hipError_t launch_filtered_r(int lg, int L, dim3 grid, hipStream_t s, const float *corpus, int64_t n, int d,
                             const float *queries, int64_t per_wave, const TreeLaunch &t, const FilterLaunch &f) {
    const TreeArgs ta = make_tree(t);
    const FilterArgs fa = make_filter(f);
    const dim3 block(64 * gemv_waves(64 * R));
#define RT_SHAPE(LGV, LV)                                                                                         \
    if (lg == LGV && L == LV) {                                                                                   \
        if (fa.crn)                                                                                               \
            hipLaunchKernelGGL((gemv_filtered_kernel<LGV, LV, R, true>), grid, block, 0, s, corpus, n, d,         \
                               queries, per_wave, ta, fa);                                                        \
        else                                                                                                      \
            hipLaunchKernelGGL((gemv_filtered_kernel<LGV, LV, R, false>), grid, block, 0, s, corpus, n, d,        \
                               queries, per_wave, ta, fa);                                                        \
        return hipGetLastError();                                                                                 \
    }
    RT_GEMV_SHAPES(RT_SHAPE)
#undef RT_SHAPE
    return hipErrorInvalidValue;
}

}  // namespace rt
