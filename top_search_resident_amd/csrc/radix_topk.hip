// radix_topk.hip -- exact large-K top-K over materialised score rows (gfx950).
//
// Used for batched retrieval with K above 128, where each query's scores were
// written by the MFMA scorer ("GPU-Resident Top-K for Agentic RAG", section 4:
// score, per-block selection, merge; section 9 and the K = 100 rows of the
// section 5 table show the pages' single-lane selector collapsing as K grows).
// With lists of up to 1024 entries per wave the merge networks dominate, so
// large K takes a radix route instead:
//
//   kernel 1: every workgroup histograms the top 11 bits of the order keys of
//             its share of a query row (LDS, one private histogram per wave),
//             then adds its non-zero bins into the row's global histogram;
//   kernel 2: every workgroup finds b*, the highest bin with at least K keys at
//             or above it -- the K-th largest key lies in b* -- and appends
//             every element whose bin is >= b* to the row's candidate buffer
//             (fewer than K from bins above b*, plus b*'s own population); the
//             last workgroup of the row to finish (an atomic arrival counter)
//             sorts the candidates in LDS and writes the K best, then clears
//             the histogram and counters for the next call.
//
// If the candidates do not fit the LDS sort (a row whose K-th bin is very
// crowded, e.g. many equal scores), that last workgroup instead selects exactly
// over the whole row: three more histogram passes pin the K-th largest key
// digit by digit, then it collects the keys above it and the lowest-index ties.
//
// Ranks are the same (key << 32 | ~index) packing as wave_topk.hpp, so the
// order -- larger score first, exact ties to the lower index -- is the pages'
// comparator (section 3, "Problem B").  Cross-XCD data (candidates, counters)
// moves through device-coherent atomic stores and loads.
#include "kernels.hpp"
#include "wave_topk.hpp"

namespace rt {

constexpr int kRadixBins = 2048;       // 11-bit digits
constexpr int kRadixHistThreads = 256;
constexpr int kRadixFilterThreads = 1024;
constexpr int kRadixSortCap = 8192;    // candidates sorted in LDS (64 KiB)

__device__ __forceinline__ uint32_t row_key(uint32_t bits) { return order_key_f32(__uint_as_float(bits)); }

// ---------------------------------------------------------------- kernel 1

__global__ __launch_bounds__(kRadixHistThreads) void radix_hist_kernel(const uint32_t *__restrict__ rows, int64_t ld,
                                                                     int64_t n, int64_t per_wg,
                                                                     uint32_t *__restrict__ hist) {
    __shared__ uint32_t h[kRadixHistThreads / 64][kRadixBins];
    const int seg = blockIdx.y;
    const int wv = wave_in_group();
    for (int i = threadIdx.x; i < (kRadixHistThreads / 64) * kRadixBins; i += blockDim.x) (&h[0][0])[i] = 0u;
    __syncthreads();
    const uint32_t *row = rows + (int64_t)seg * ld;
    const int64_t begin = (int64_t)blockIdx.x * per_wg;  // per_wg is a multiple of 4 and ld of 64: 16-byte aligned
    const int64_t end = (begin + per_wg < n) ? begin + per_wg : n;
    for (int64_t e = begin + 4 * (int64_t)threadIdx.x; e < end; e += 4 * (int64_t)blockDim.x) {
        const uint4 v = *reinterpret_cast<const uint4 *>(row + e);
        const uint32_t x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (e + c < end) atomicAdd(&h[wv][row_key(x[c]) >> 21], 1u);
    }
    __syncthreads();
    for (int b = threadIdx.x; b < kRadixBins; b += blockDim.x) {
        uint32_t c = 0;
#pragma unroll
        for (int w = 0; w < kRadixHistThreads / 64; ++w) c += h[w][b];
        if (c) atomicAdd(&hist[(int64_t)seg * kRadixBins + b], c);
    }
}

// ---------------------------------------------------------------- kernel 2 helpers

// Inclusive prefix sum of one value per thread over the workgroup (LDS scratch
// `buf` of blockDim entries).  Returns this thread's inclusive sum.
__device__ __forceinline__ uint32_t block_inclusive_scan(uint32_t v, uint32_t *buf) {
    const int t = threadIdx.x;
    buf[t] = v;
    __syncthreads();
    for (int off = 1; off < (int)blockDim.x; off <<= 1) {
        const uint32_t add = (t >= off) ? buf[t - off] : 0u;
        __syncthreads();
        buf[t] += add;
        __syncthreads();
    }
    const uint32_t r = buf[t];
    __syncthreads();
    return r;
}

// Sort sm[0..m) (m a power of two) best-first.
__device__ __forceinline__ void lds_bitonic_sort_desc(uint64_t *sm, int m) {
    for (int k2 = 2; k2 <= m; k2 <<= 1) {
        for (int j = k2 >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < m; i += blockDim.x) {
                const int p = i ^ j;
                if (p > i) {
                    const uint64_t a = sm[i], b = sm[p];
                    const bool desc = (i & k2) == 0;
                    if (desc ? (a < b) : (a > b)) {
                        sm[i] = b;
                        sm[p] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
}

struct RadixOut {
    int k;
    int32_t *out_idx;  // [segments][k]
    uint32_t *out_val; // [segments][k], fp32 scores from the ranks
};

__device__ __forceinline__ void radix_write(const RadixOut &o, int seg, int r, uint64_t v) {
    o.out_idx[(int64_t)seg * o.k + r] = (int32_t)rank_index(v);
    o.out_val[(int64_t)seg * o.k + r] = __float_as_uint(f32_of_order_key(rank_key(v)));
}

// Exact top-k of one whole row by one workgroup: pin the k-th largest key with
// three histogram passes (11 + 11 + 10 bits), then collect every key above it
// and, in index order, the lowest-index elements equal to it.
__device__ void select_row_exactly(const uint32_t *row, int64_t n, const RadixOut &o, int seg, uint64_t *sm,
                                   uint32_t *sh, uint32_t *scan_buf, uint32_t *s_vals) {
    uint32_t prefix = 0, pmask = 0;
    uint32_t need = (uint32_t)o.k;  // how many of the remaining keys to take from the top
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
    for (int pass = 0; pass < 3; ++pass) {
        const int sh_bits = shifts[pass];
        const uint32_t dmask = (1u << widths[pass]) - 1u;
        for (int b = threadIdx.x; b < kRadixBins; b += blockDim.x) sh[b] = 0u;
        __syncthreads();
        for (int64_t e = threadIdx.x; e < n; e += blockDim.x) {
            const uint32_t key = row_key(row[e]);
            if ((key & pmask) == prefix) atomicAdd(&sh[(key >> sh_bits) & dmask], 1u);
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t cum = 0;
            int digit = 0;
            for (int b = (int)dmask; b >= 0; --b) {
                if (cum + sh[b] >= need) {
                    digit = b;
                    break;
                }
                cum += sh[b];
            }
            s_vals[0] = prefix | ((uint32_t)digit << sh_bits);
            s_vals[1] = need - cum;
        }
        __syncthreads();
        prefix = s_vals[0];
        need = s_vals[1];
        pmask |= dmask << sh_bits;
        __syncthreads();
    }
    const uint32_t T = prefix;         // the k-th largest key
    const uint32_t ties = need;        // how many keys equal to T belong to the top-k
    if (threadIdx.x == 0) s_vals[2] = 0u;
    __syncthreads();
    for (int64_t e = threadIdx.x; e < n; e += blockDim.x) {
        const uint32_t key = row_key(row[e]);
        if (key > T) sm[atomicAdd(&s_vals[2], 1u)] = make_rank(key, (uint32_t)e);
    }
    __syncthreads();
    uint32_t taken = 0;  // ties collected so far, identical in every thread
    for (int64_t c0 = 0; c0 < n && taken < ties; c0 += blockDim.x) {
        const int64_t e = c0 + threadIdx.x;
        const bool eq = e < n && row_key(row[e]) == T;
        const uint32_t incl = block_inclusive_scan(eq ? 1u : 0u, scan_buf);
        const uint32_t ordinal = taken + incl - (eq ? 1u : 0u);
        if (eq && ordinal < ties) sm[o.k - ties + ordinal] = make_rank(T, (uint32_t)e);
        taken += scan_buf[blockDim.x - 1];  // the chunk's total: the last thread's inclusive sum
        __syncthreads();
    }
    int m = 64;
    while (m < o.k) m <<= 1;
    for (int i = o.k + threadIdx.x; i < m; i += blockDim.x) sm[i] = 0ull;
    __syncthreads();
    lds_bitonic_sort_desc(sm, m);
    for (int r = threadIdx.x; r < o.k; r += blockDim.x) radix_write(o, seg, r, sm[r]);
}

// ---------------------------------------------------------------- kernel 2

__global__ __launch_bounds__(kRadixFilterThreads) void radix_filter_kernel(
    const uint32_t *__restrict__ rows, int64_t ld, int64_t n, int64_t per_wg, uint32_t *__restrict__ hist,
    uint32_t *__restrict__ ccount, uint64_t *__restrict__ cand, int64_t capc, uint32_t *__restrict__ arrive,
    RadixOut o) {
    __shared__ uint64_t sm[kRadixSortCap];
    __shared__ uint32_t sh[kRadixBins];
    __shared__ uint32_t scan_buf[kRadixFilterThreads];
    __shared__ uint32_t s_vals[4];
    const int seg = blockIdx.y;
    const int t = threadIdx.x;
    const int lane = lane_id();
    uint32_t *h = hist + (int64_t)seg * kRadixBins;
    const uint32_t *row = rows + (int64_t)seg * ld;

    // b*: the highest bin whose suffix count (bins >= it) reaches k.  Thread t
    // owns bins 2047 - 2t and 2046 - 2t; a prefix sum over threads gives the
    // suffix counts in descending bin order.
    const uint32_t hi = h[kRadixBins - 1 - 2 * t];
    const uint32_t lo = h[kRadixBins - 2 - 2 * t];
    const uint32_t incl = block_inclusive_scan(hi + lo, scan_buf);
    const uint32_t before = incl - hi - lo;
    if (before < (uint32_t)o.k && incl >= (uint32_t)o.k)
        s_vals[0] = (before + hi >= (uint32_t)o.k) ? (uint32_t)(kRadixBins - 1 - 2 * t) : (uint32_t)(kRadixBins - 2 - 2 * t);
    __syncthreads();
    const uint32_t bstar = s_vals[0];

    // Append every element whose bin is >= b*.  Candidates are staged in LDS
    // (sm, reused later for the final sort) behind a workgroup-local counter, and
    // the workgroup reserves its slice of the row's buffer with one global
    // atomic at the end: a returning device atomic per wave step on one counter
    // per row serialised to ~0.5 ms per call at 32 x 500k.  Overflow past the
    // LDS capacity (crowded bins) goes straight to the global buffer.
    const int64_t begin = (int64_t)blockIdx.x * per_wg;
    const int64_t end = (begin + per_wg < n) ? begin + per_wg : n;
    uint32_t *cnt = &ccount[seg];
    uint64_t *cbuf = cand + (int64_t)seg * capc;
    if (t == 0) s_vals[2] = 0u;
    __syncthreads();
    for (int64_t e0 = begin; e0 < end; e0 += 4 * (int64_t)blockDim.x) {
        const int64_t e = e0 + 4 * (int64_t)t;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (e < end) v = *reinterpret_cast<const uint4 *>(row + e);
        const uint32_t x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t key = row_key(x[c]);
            const bool take = (e + c < end) && (key >> 21) >= bstar;
            const uint64_t m = __ballot(take);
            if (m == 0) continue;
            uint32_t base = 0;
            if (lane == 0) base = atomicAdd(&s_vals[2], (uint32_t)__popcll(m));
            base = (uint32_t)__shfl(base, 0);
            const uint32_t pos = base + (uint32_t)lanes_below(m);
            if (take) {
                const uint64_t rank = make_rank(key, (uint32_t)(e + c));
                if (pos < (uint32_t)kRadixSortCap) {
                    sm[pos] = rank;
                } else {
                    const uint32_t gpos = atomicAdd(cnt, 1u);
                    if ((int64_t)gpos < capc)
                        __hip_atomic_store(&cbuf[gpos], rank, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
    }
    __syncthreads();
    const uint32_t staged = (s_vals[2] < (uint32_t)kRadixSortCap) ? s_vals[2] : (uint32_t)kRadixSortCap;
    if (t == 0) s_vals[3] = staged ? atomicAdd(cnt, staged) : 0u;
    __syncthreads();
    const uint32_t gbase = s_vals[3];
    for (uint32_t i = t; i < staged; i += blockDim.x)
        if ((int64_t)(gbase + i) < capc)
            __hip_atomic_store(&cbuf[gbase + i], sm[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // the last workgroup of this row finishes it
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t == 0) {
        const uint32_t arrived = atomicAdd(&arrive[seg], 1u);
        const uint32_t last = (arrived + 1 == gridDim.x) ? 1u : 0u;
        if (last) __hip_atomic_store(&arrive[seg], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_vals[1] = last;
    }
    __syncthreads();
    if (!s_vals[1]) return;
    const uint32_t total = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (total <= (uint32_t)kRadixSortCap && (int64_t)total <= capc) {
        int m = 64;
        while (m < (int)total) m <<= 1;
        for (int i = t; i < m; i += blockDim.x)
            sm[i] = (i < (int)total) ? __hip_atomic_load(&cbuf[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0ull;
        __syncthreads();
        lds_bitonic_sort_desc(sm, m);
        for (int r = t; r < o.k; r += blockDim.x) radix_write(o, seg, r, sm[r]);
    } else {
        select_row_exactly(row, n, o, seg, sm, sh, scan_buf, s_vals);
    }
    // clear this row's histogram and candidate count for the next call
    for (int b = t; b < kRadixBins; b += blockDim.x)
        __hip_atomic_store(&h[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (t == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- launcher

hipError_t launch_radix_topk(const float *rows, int64_t ld, int64_t n, int segments, int k, int wgs_per_seg,
                             const RadixScratch &sc, int32_t *out_idx, float *out_scores, hipStream_t stream) {
    int64_t per_wg = (n + wgs_per_seg - 1) / wgs_per_seg;
    per_wg = (per_wg + 3) / 4 * 4;
    const int wgs = (int)((n + per_wg - 1) / per_wg);
    const uint32_t *r = reinterpret_cast<const uint32_t *>(rows);
    hipLaunchKernelGGL(radix_hist_kernel, dim3(wgs, segments), dim3(kRadixHistThreads), 0, stream, r, ld, n, per_wg,
                       sc.hist);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    RadixOut o;
    o.k = k;
    o.out_idx = out_idx;
    o.out_val = reinterpret_cast<uint32_t *>(out_scores);
    hipLaunchKernelGGL(radix_filter_kernel, dim3(wgs, segments), dim3(kRadixFilterThreads), 0, stream, r, ld, n,
                       per_wg, sc.hist, sc.count, sc.cand, sc.cand_cap, sc.arrive, o);
    return hipGetLastError();
}

}  // namespace rt
