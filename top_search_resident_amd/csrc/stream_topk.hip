// stream_topk.hip -- the streaming stage of exact top-K on gfx950.
//
// "GPU-Resident Top-K for Agentic RAG" (A. Banerjee), section 4: Step 2 scores
// every corpus row by inner product, Step 3 lets each block of rows build its own
// best-K list.  The pages run one thread per row for scoring (uncoalesced along
// D) and a single-lane bubble sort per block for selection; here one kernel does
// both: each wavefront streams a contiguous row range with 16-byte coalesced
// loads, reduces each row's dot product across a group of lanes, and feeds the
// scores straight into a register-resident best-K list (wave_topk.hpp), so the
// N scores never go to HBM.  At the end the four waves of a workgroup merge their
// lists into one list per workgroup.
//
// The raw-array variant is the first stage of the two-stage top-K of "CUDA
// Programming Model Series 9: Efficient TopK" (section 2: each block reduces its
// share of the array to a local top-K), with vectorised loads and the same
// register lists.
#include "kernels.hpp"
#include "wave_topk.hpp"

namespace rt {

// Rows per lane-group step unrolled so each lane keeps ~8 float4 loads in flight.
template <int L>
struct RowUnroll {
    static constexpr int value = (L >= 6) ? 1 : (L >= 3 ? 2 : (L == 2 ? 4 : 8));
};

// Write the 4 waves' lists to LDS, merge them pairwise, store the workgroup's
// list (best-first, Kp entries) to `out`.
template <int R>
__device__ __forceinline__ void workgroup_merge_store(WaveSelector<R> &sel, uint64_t *lds, uint64_t *out) {
    constexpr int Kp = 64 * R;
    const int lane = lane_id();
    const int wv = threadIdx.x >> 6;
#pragma unroll
    for (int r = 0; r < R; ++r) lds[wv * Kp + r * 64 + lane] = sel.L[r];
    __syncthreads();
    if ((wv & 1) == 0) {
        uint64_t M[R];
#pragma unroll
        for (int r = 0; r < R; ++r) M[r] = lds[(wv + 1) * Kp + r * 64 + lane];
        list_absorb_list<R>(sel.L, M);
#pragma unroll
        for (int r = 0; r < R; ++r) lds[wv * Kp + r * 64 + lane] = sel.L[r];
    }
    __syncthreads();
    if (wv == 0) {
        uint64_t M[R];
#pragma unroll
        for (int r = 0; r < R; ++r) M[r] = lds[2 * Kp + r * 64 + lane];
        list_absorb_list<R>(sel.L, M);
#pragma unroll
        for (int r = 0; r < R; ++r) out[r * 64 + lane] = sel.L[r];
    }
}

// ---------------------------------------------------------------- scoring

// A group of G = 2^log2g lanes owns one row at a time; lane g of the group loads
// float4 columns g, g+G, ..., g+(L-1)G of that row (masked past d/4), so a row is
// covered by one instruction per j and consecutive lanes read consecutive 16 B.
// Every row is reduced in exactly the same order (per-lane FMA chain over j and
// the four components, then an xor butterfly over the group), so identical rows
// get bit-identical scores wherever they sit, and exact ties resolve by index.
template <int L, int R>
__global__ __launch_bounds__(kStreamThreads) void gemv_topk_kernel(
    const float *__restrict__ corpus, int64_t n, int d, int log2g, const float *__restrict__ queries,
    int64_t rows_per_wave, int k, uint64_t *__restrict__ wg_lists, uint64_t *__restrict__ seg_thr) {
    constexpr int U = RowUnroll<L>::value;
    constexpr int Kp = 64 * R;
    __shared__ uint64_t stage[kStreamWaves][128];
    __shared__ uint64_t lists[kStreamWaves * Kp];

    const int seg = blockIdx.y;
    const int lane = lane_id();
    const int wv = threadIdx.x >> 6;
    const int64_t wave = (int64_t)blockIdx.x * kStreamWaves + wv;
    const int G = 1 << log2g;
    const int g = lane & (G - 1);
    const int h = lane >> log2g;
    const int rps = 64 >> log2g;
    const int d4 = d >> 2;
    const float4 *__restrict__ c4 = reinterpret_cast<const float4 *>(corpus);
    const float4 *__restrict__ q4 = reinterpret_cast<const float4 *>(queries + (int64_t)seg * d);

    WaveSelector<R> sel;
    sel.init(k);
    uint64_t *const my_stage = stage[wv];
    uint64_t *const my_thr = seg_thr + seg;

    float4 qv[L];
#pragma unroll
    for (int j = 0; j < L; ++j) {
        const int col = j * G + g;
        qv[j] = (col < d4) ? q4[col] : make_float4(0.f, 0.f, 0.f, 0.f);
    }

    const int64_t r_begin = wave * rows_per_wave;
    const int64_t r_end = (r_begin + rows_per_wave < n) ? r_begin + rows_per_wave : n;
    for (int64_t r0 = r_begin; r0 < r_end; r0 += (int64_t)rps * U) {
        float4 x[U][L];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = r0 + u * rps + h;
            const bool ok = row < r_end;
            const float4 *rp = c4 + row * d4;
#pragma unroll
            for (int j = 0; j < L; ++j) {
                const int col = j * G + g;
                x[u][j] = (ok && col < d4) ? rp[col] : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        sel.refresh(my_thr);
        float acc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float a = 0.f;
#pragma unroll
            for (int j = 0; j < L; ++j) {
                a = fmaf(x[u][j].x, qv[j].x, a);
                a = fmaf(x[u][j].y, qv[j].y, a);
                a = fmaf(x[u][j].z, qv[j].z, a);
                a = fmaf(x[u][j].w, qv[j].w, a);
            }
            acc[u] = a;
        }
        for (int m = G >> 1; m >= 1; m >>= 1) {
#pragma unroll
            for (int u = 0; u < U; ++u) acc[u] += __shfl_xor(acc[u], m);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = r0 + u * rps + h;
            const bool valid = (g == 0) && (row < r_end);
            const uint64_t rank = make_rank(order_key_f32(acc[u]), (uint32_t)row);
            sel.offer(my_stage, my_thr, rank, valid && rank > sel.thr);
        }
    }
    sel.finish(my_stage, my_thr);
    workgroup_merge_store<R>(sel, lists, wg_lists + ((int64_t)seg * gridDim.x + blockIdx.x) * Kp);
}

// Any d: one row per wave at a time, scalar loads strided by 64 lanes.
template <int R>
__global__ __launch_bounds__(kStreamThreads) void gemv_topk_generic_kernel(
    const float *__restrict__ corpus, int64_t n, int d, const float *__restrict__ queries,
    int64_t rows_per_wave, int k, uint64_t *__restrict__ wg_lists, uint64_t *__restrict__ seg_thr) {
    constexpr int Kp = 64 * R;
    constexpr int U = 4;
    __shared__ uint64_t stage[kStreamWaves][128];
    __shared__ uint64_t lists[kStreamWaves * Kp];
    const int seg = blockIdx.y;
    const int lane = lane_id();
    const int wv = threadIdx.x >> 6;
    const int64_t wave = (int64_t)blockIdx.x * kStreamWaves + wv;
    const float *__restrict__ q = queries + (int64_t)seg * d;
    WaveSelector<R> sel;
    sel.init(k);
    uint64_t *const my_stage = stage[wv];
    uint64_t *const my_thr = seg_thr + seg;
    const int64_t r_begin = wave * rows_per_wave;
    const int64_t r_end = (r_begin + rows_per_wave < n) ? r_begin + rows_per_wave : n;
    for (int64_t r0 = r_begin; r0 < r_end; r0 += U) {
        float acc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) acc[u] = 0.f;
        for (int c = lane; c < d; c += 64) {
            const float qc = q[c];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t row = r0 + u;
                const float x = (row < r_end) ? corpus[row * d + c] : 0.f;
                acc[u] = fmaf(x, qc, acc[u]);
            }
        }
        sel.refresh(my_thr);
        for (int m = 32; m >= 1; m >>= 1) {
#pragma unroll
            for (int u = 0; u < U; ++u) acc[u] += __shfl_xor(acc[u], m);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = r0 + u;
            const bool valid = (lane == 0) && (row < r_end);
            const uint64_t rank = make_rank(order_key_f32(acc[u]), (uint32_t)row);
            sel.offer(my_stage, my_thr, rank, valid && rank > sel.thr);
        }
    }
    sel.finish(my_stage, my_thr);
    workgroup_merge_store<R>(sel, lists, wg_lists + ((int64_t)seg * gridDim.x + blockIdx.x) * Kp);
}

// ---------------------------------------------------------------- raw arrays

// Segment `seg` is the n-element array at base + seg * seg_stride (32-bit
// elements).  It is read as 16-byte groups of the enclosing aligned range: group
// t holds elements 4t - head .. 4t - head + 3, where head = (address mod 16) / 4.
// Elements outside [0, n) are masked.  An aligned 16-byte group never crosses a
// page, so reading the part of a group outside the array cannot fault.
template <int DT, int R>
__global__ __launch_bounds__(kStreamThreads) void select_topk_kernel(
    const uint32_t *__restrict__ base, int64_t seg_stride, int64_t n, int64_t groups_per_wave, int k,
    uint64_t *__restrict__ wg_lists, uint64_t *__restrict__ seg_thr) {
    constexpr int Kp = 64 * R;
    constexpr int U = 4;
    __shared__ uint64_t stage[kStreamWaves][128];
    __shared__ uint64_t lists[kStreamWaves * Kp];
    const int seg = blockIdx.y;
    const int lane = lane_id();
    const int wv = threadIdx.x >> 6;
    const int64_t wave = (int64_t)blockIdx.x * kStreamWaves + wv;
    const uintptr_t addr = reinterpret_cast<uintptr_t>(base + seg * seg_stride);
    const int head = (int)((addr & 15u) >> 2);
    const uint4 *__restrict__ a4 = reinterpret_cast<const uint4 *>(addr - (uintptr_t)head * 4u);
    const int64_t total_groups = (n + head + 3) >> 2;

    WaveSelector<R> sel;
    sel.init(k);
    uint64_t *const my_stage = stage[wv];
    uint64_t *const my_thr = seg_thr + seg;
    const int64_t g_begin = wave * groups_per_wave;
    const int64_t g_end = (g_begin + groups_per_wave < total_groups) ? g_begin + groups_per_wave : total_groups;
    for (int64_t g0 = g_begin; g0 < g_end; g0 += 64 * U) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t grp = g0 + u * 64 + lane;
            v[u] = (grp < g_end) ? a4[grp] : make_uint4(0u, 0u, 0u, 0u);
        }
        sel.refresh(my_thr);
        uint32_t key[U][4];
        bool any = false;
        const uint32_t thr_key = rank_key(sel.thr);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
            const int64_t grp = g0 + u * 64 + lane;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                key[u][c] = (DT == 0) ? order_key_i32((int32_t)e[c]) : order_key_f32(__uint_as_float(e[c]));
                const int64_t idx = grp * 4 + c - head;
                const bool valid = (grp < g_end) && idx >= 0 && idx < n;
                any |= valid && key[u][c] >= thr_key;
            }
        }
        if (__ballot(any) == 0) continue;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t grp = g0 + u * 64 + lane;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int64_t idx = grp * 4 + c - head;
                const bool valid = (grp < g_end) && idx >= 0 && idx < n;
                const uint64_t rank = make_rank(key[u][c], (uint32_t)idx);
                sel.offer(my_stage, my_thr, rank, valid && rank > sel.thr);
            }
        }
    }
    sel.finish(my_stage, my_thr);
    workgroup_merge_store<R>(sel, lists, wg_lists + ((int64_t)seg * gridDim.x + blockIdx.x) * Kp);
}

// ---------------------------------------------------------------- launchers

bool gemv_fast_path_ok(int d) { return d % 4 == 0 && d / 4 <= 64 * 8; }

// Pick the lane-group width G (power of two <= 64) and loads per lane L (from
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

template <int L>
static hipError_t gemv_by_r(int R, dim3 grid, hipStream_t s, const float *corpus, int64_t n, int d, int lg,
                            const float *q, int64_t rpw, int k, uint64_t *lists, uint64_t *thr) {
    switch (R) {
#define RT_CASE(RR)                                                                                          \
    case RR:                                                                                                 \
        hipLaunchKernelGGL((gemv_topk_kernel<L, RR>), grid, dim3(kStreamThreads), 0, s, corpus, n, d, lg, q, \
                           rpw, k, lists, thr);                                                              \
        break;
        RT_CASE(1) RT_CASE(2) RT_CASE(4) RT_CASE(8) RT_CASE(16)
#undef RT_CASE
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gemv_topk(const float *corpus, int64_t n, int d, const float *queries, int segments, int k,
                            int kp, int64_t rows_per_wave, int wgs_per_seg, uint64_t *wg_lists,
                            uint64_t *seg_thr, hipStream_t stream) {
    const int R = kp / 64;
    const dim3 grid(wgs_per_seg, segments);
    if (!gemv_fast_path_ok(d)) {
        switch (R) {
#define RT_CASE(RR)                                                                                            \
    case RR:                                                                                                   \
        hipLaunchKernelGGL((gemv_topk_generic_kernel<RR>), grid, dim3(kStreamThreads), 0, stream, corpus, n, d, \
                           queries, rows_per_wave, k, wg_lists, seg_thr);                                      \
        break;
            RT_CASE(1) RT_CASE(2) RT_CASE(4) RT_CASE(8) RT_CASE(16)
#undef RT_CASE
            default:
                return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    int lg = 6, L = 8;
    pick_group(d / 4, &lg, &L);
    switch (L) {
        case 1: return gemv_by_r<1>(R, grid, stream, corpus, n, d, lg, queries, rows_per_wave, k, wg_lists, seg_thr);
        case 2: return gemv_by_r<2>(R, grid, stream, corpus, n, d, lg, queries, rows_per_wave, k, wg_lists, seg_thr);
        case 3: return gemv_by_r<3>(R, grid, stream, corpus, n, d, lg, queries, rows_per_wave, k, wg_lists, seg_thr);
        case 4: return gemv_by_r<4>(R, grid, stream, corpus, n, d, lg, queries, rows_per_wave, k, wg_lists, seg_thr);
        case 6: return gemv_by_r<6>(R, grid, stream, corpus, n, d, lg, queries, rows_per_wave, k, wg_lists, seg_thr);
        case 8: return gemv_by_r<8>(R, grid, stream, corpus, n, d, lg, queries, rows_per_wave, k, wg_lists, seg_thr);
        default: return hipErrorInvalidValue;
    }
}

template <int DT>
static hipError_t select_by_r(int R, dim3 grid, hipStream_t s, const uint32_t *base, int64_t stride, int64_t n,
                              int64_t gpw, int k, uint64_t *lists, uint64_t *thr) {
    switch (R) {
#define RT_CASE(RR)                                                                                           \
    case RR:                                                                                                  \
        hipLaunchKernelGGL((select_topk_kernel<DT, RR>), grid, dim3(kStreamThreads), 0, s, base, stride, n, gpw, \
                           k, lists, thr);                                                                    \
        break;
        RT_CASE(1) RT_CASE(2) RT_CASE(4) RT_CASE(8) RT_CASE(16)
#undef RT_CASE
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_select_topk(const void *base, int64_t seg_stride, int64_t n, int dtype, int segments, int k,
                              int kp, int64_t groups_per_wave, int wgs_per_seg, uint64_t *wg_lists,
                              uint64_t *seg_thr, hipStream_t stream) {
    const dim3 grid(wgs_per_seg, segments);
    const uint32_t *b = static_cast<const uint32_t *>(base);
    if (dtype == 0) return select_by_r<0>(kp / 64, grid, stream, b, seg_stride, n, groups_per_wave, k, wg_lists, seg_thr);
    if (dtype == 1) return select_by_r<1>(kp / 64, grid, stream, b, seg_stride, n, groups_per_wave, k, wg_lists, seg_thr);
    return hipErrorInvalidValue;
}

}  // namespace rt
