// batch_select.hip -- exact top-K of materialised batch score rows (gfx950).
//
// Batched retrieval writes each query's scores to a row of S and, per query,
// the largest score of every 32-row tile (mfma_scores.hip).  The pages score
// one query at a time and select with one lane per block ("GPU-Resident Top-K
// for Agentic RAG", section 4 Steps 3-4; section 9 and the K = 100 rows of the
// section 5 table show that selector collapsing as K grows).  Here K tiles
// whose maxima reach a value B hold K distinct scores >= B, so the K-th score
// is >= B: one workgroup per query pins the K-th largest tile maximum to a
// narrow bin, reads only the tiles that reach its lower edge (about K tiles),
// keeps their scores at or above it and sorts those.  If too many tiles or
// scores qualify (many equal scores), the workgroup selects exactly over the
// whole row instead: three histogram passes pin the K-th largest key digit by
// digit, then it collects the keys above it and the lowest-index ties.
//
// Ranks are the same (key << 32 | ~index) packing as wave_topk.hpp, so the
// order -- larger score first, exact ties to the lower index -- is the pages'
// comparator (section 3, "Problem B").
#include "block_sort.hpp"
#include "kernels.hpp"
#include "wave_topk.hpp"

namespace rt {

constexpr int kDigitBins = 2048;       // 11-bit digits
constexpr int kBatchSelectThreads = 1024;
constexpr int kSortCap = 8192;    // candidates sorted in LDS (64 KiB)

__device__ __forceinline__ uint32_t row_key(uint32_t bits) { return order_key_f32(__uint_as_float(bits)); }

// ---------------------------------------------------------------- helpers

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

// Sort sm[0 .. m) best-first, m a power of two in [64, kSortCap].
__device__ __forceinline__ void block_sort_desc(uint64_t *sm, int m) {
    block_sort_desc_any<kBatchSelectThreads, kSortCap>(sm, m);
}

struct SelectOut {
    int k;
    int32_t *out_idx;  // [segments][k]
    uint32_t *out_val; // [segments][k], fp32 scores from the ranks
};

__device__ __forceinline__ void write_result(const SelectOut &o, int seg, int r, uint64_t v) {
    o.out_idx[(int64_t)seg * o.k + r] = (int32_t)rank_index(v);
    o.out_val[(int64_t)seg * o.k + r] = __float_as_uint(f32_of_order_key(rank_key(v)));
}

// Exact top-k of one whole row by one workgroup: pin the k-th largest key with
// three histogram passes (11 + 11 + 10 bits), then collect every key above it
// and, in index order, the lowest-index elements equal to it.
__device__ void select_row_exactly(const uint32_t *row, int64_t n, const SelectOut &o, int seg, uint64_t *sm,
                                   uint32_t *sh, uint32_t *scan_buf, uint32_t *s_vals) {
    uint32_t prefix = 0, pmask = 0;
    uint32_t need = (uint32_t)o.k;  // how many of the remaining keys to take from the top
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
    for (int pass = 0; pass < 3; ++pass) {
        const int sh_bits = shifts[pass];
        const uint32_t dmask = (1u << widths[pass]) - 1u;
        for (int b = threadIdx.x; b < kDigitBins; b += blockDim.x) sh[b] = 0u;
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
    block_sort_desc(sm, m);
    for (int r = threadIdx.x; r < o.k; r += blockDim.x) write_result(o, seg, r, sm[r]);
}

// ---------------------------------------------------------------- tile-bounded selection

// Top-k of score rows that come with per-tile maxima (tmax[row][tile] = largest
// score among elements 32 tile .. 32 tile + 31).  K tiles whose maxima reach a
// value B hold K distinct elements >= B, so the k-th largest score is >= B and
// every element of the top k lies in a tile whose maximum is >= B.  One
// workgroup per row:
//   1. histograms of the tile-maximum keys pin the k-th largest one to a bin
//      (see below); B is the lower edge of that bin, so at least k tiles
//      reach it;
//   2. the tiles whose maximum reaches B are listed (about k of them for
//      i.i.d. scores), their scores read, and those >= B kept in LDS;
//   3. the kept ranks are sorted in LDS and the best k written.
// A row with fewer than k tiles keeps every element; if the tile list or the
// kept ranks overflow LDS (many equal scores), the row is selected exactly by
// select_row_exactly instead.
constexpr int kTileListCap = 4096;

// Call f(i, in_range, key) for tile maxima i = 0 .. tiles - 1, thread by thread
// in blocks of 16 per thread whose loads are all issued before any is used.
// Every lane calls f the same number of times (f may use wave ballots).  The
// loads are unconditional (clamped index) and all keys are formed before any
// f runs: a load or a use inside a branch makes the compiler wait for every
// outstanding load there.
template <typename F>
__device__ __forceinline__ void scan_tiles(const uint32_t *tm, int64_t tiles, F &&f) {
    constexpr int U = 16;
    for (int64_t i0 = 0; i0 < tiles; i0 += (int64_t)U * blockDim.x) {
        uint32_t kv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = i0 + (int64_t)u * blockDim.x + threadIdx.x;
            kv[u] = tm[i < tiles ? i : tiles - 1];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) kv[u] = row_key(kv[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = i0 + (int64_t)u * blockDim.x + threadIdx.x;
            f(i, i < tiles, kv[u]);
        }
    }
}

// One segment's tile maxima as keys for the scans below: read once into
// registers when they fit (tiles <= 16 per thread: every batched workload up
// to 16,384 tiles, 524,288 rows), so the two or three scans of a call read
// global memory once; otherwise each scan re-reads them (scan_tiles).
struct TileKeys {
    static constexpr int U = 16;
    uint32_t kv[U];
    const uint32_t *tm;
    int64_t tiles;
    bool cached;
    __device__ __forceinline__ void load(const uint32_t *tm_, int64_t tiles_) {
        tm = tm_;
        tiles = tiles_;
        cached = tiles <= (int64_t)U * blockDim.x;  // uniform over the workgroup
        if (cached) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = (int64_t)u * blockDim.x + threadIdx.x;
                kv[u] = tm[i < tiles ? i : tiles - 1];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) kv[u] = row_key(kv[u]);
        }
    }
    // f(i, i < tiles, key of tile i), the same number of calls on every lane
    template <typename F>
    __device__ __forceinline__ void for_each(F &&f) const {
        if (cached) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = (int64_t)u * blockDim.x + threadIdx.x;
                f(i, i < tiles, kv[u]);
            }
        } else {
            scan_tiles(tm, tiles, f);
        }
    }
};

// Step 1 of tile_bound_select_kernel below, for the rows' tile maxima tm[0 ..
// tiles): the lower edge of a key bin that holds the k-th largest tile
// maximum, so at least k tiles reach it (as a key; 0, below every key, when
// there are fewer than k tiles).  Every thread of the workgroup calls it and
// gets the same value.  Tile maxima crowd into a few top-11-bit bins, so the
// first try histograms a window just below the largest tile maximum in 2048
// bins of 2^12 key units (2^23 units: one octave for fp32), counting only keys
// inside it: few keys, spread out, few LDS collisions.  If fewer than k keys
// fall inside, two plain 11-bit passes over all keys pin the top 22 bits
// instead.
__device__ uint32_t tile_max_bound(const TileKeys &keys, int k, uint32_t *sh, uint32_t *scan_buf,
                                   uint32_t *s_vals) {
    const int64_t tiles = keys.tiles;
    const int t = threadIdx.x;
    const int lane = lane_id();
    uint32_t bound = 0;
    if (tiles >= k) {
        uint32_t top = 0;
        keys.for_each([&](int64_t, bool ok, uint32_t key) {
            if (ok) top = max(top, key);
        });
        for (int off = 32; off >= 1; off >>= 1) top = max(top, (uint32_t)__shfl_xor((int)top, off));
        if (t == 0) {
            s_vals[0] = 0u;
            s_vals[1] = 0xffffffffu;
        }
        for (int b = t; b < kDigitBins; b += blockDim.x) sh[b] = 0u;
        __syncthreads();
        if (lane == 0) atomicMax(&s_vals[0], top);
        __syncthreads();
        top = s_vals[0] >> 12;  // window: key >> 12 in (top - 2048, top]
        keys.for_each([&](int64_t, bool ok, uint32_t key) {
            const uint32_t dist = top - (key >> 12);
            if (ok && dist < (uint32_t)kDigitBins) atomicAdd(&sh[dist], 1u);
        });
        __syncthreads();
        // lowest window bin (distance from the top) whose prefix count reaches
        // k, found by one wave: lane l sums bins 32 l .. 32 l + 31, a wave
        // prefix sum finds the lane whose range holds it, that lane walks its
        // bins (one workgroup barrier instead of a block-wide scan)
        if (t < 64) {
            constexpr int B = kDigitBins / 64;
            uint32_t c[B];
            uint32_t sum = 0;
#pragma unroll
            for (int i = 0; i < B; ++i) {
                c[i] = sh[B * t + i];
                sum += c[i];
            }
            uint32_t incl = sum;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t y = __shfl_up(incl, off, 64);
                if (t >= off) incl += y;
            }
            uint32_t before = incl - sum;
            if (before < (uint32_t)k && incl >= (uint32_t)k) {
                uint32_t found = 0xffffffffu;
#pragma unroll
                for (int i = 0; i < B; ++i) {
                    if (found == 0xffffffffu) {
                        if (before + c[i] >= (uint32_t)k)
                            found = (uint32_t)(B * t + i);
                        else
                            before += c[i];
                    }
                }
                s_vals[1] = found;
            }
        }
        __syncthreads();
        const uint32_t dist = s_vals[1];
        if (dist != 0xffffffffu) {
            bound = (top - dist) << 12;
        } else {
            uint32_t prefix = 0, pmask = 0, need = (uint32_t)k;
            for (int pass = 0; pass < 2; ++pass) {
                const int shift = pass == 0 ? 21 : 10;
                for (int b = t; b < kDigitBins; b += blockDim.x) sh[b] = 0u;
                __syncthreads();
                keys.for_each([&](int64_t, bool ok, uint32_t key) {
                    if (ok && (key & pmask) == prefix) atomicAdd(&sh[(key >> shift) & (kDigitBins - 1)], 1u);
                });
                __syncthreads();
                // highest digit whose suffix count reaches `need`: thread t
                // owns digits 2047 - 2t and 2046 - 2t, a prefix sum gives
                // suffix counts
                const uint32_t hi = sh[kDigitBins - 1 - 2 * t];
                const uint32_t lo = sh[kDigitBins - 2 - 2 * t];
                const uint32_t incl2 = block_inclusive_scan(hi + lo, scan_buf);
                const uint32_t before2 = incl2 - hi - lo;
                if (before2 < need && incl2 >= need) {
                    const bool in_hi = before2 + hi >= need;
                    s_vals[0] = (uint32_t)(kDigitBins - (in_hi ? 1 : 2) - 2 * t);
                    s_vals[1] = in_hi ? before2 : before2 + hi;  // keys above the digit
                }
                __syncthreads();
                prefix |= s_vals[0] << shift;
                need -= s_vals[1];
                pmask |= (uint32_t)(kDigitBins - 1) << shift;
                __syncthreads();
            }
            bound = prefix;
        }
    }
    return bound;
}

__global__ __launch_bounds__(kBatchSelectThreads) void tile_bound_select_kernel(const uint32_t *__restrict__ rows,
                                                                              int64_t ld, int64_t n,
                                                                              const uint32_t *__restrict__ tmax,
                                                                              int64_t tld, SelectOut o) {
    __shared__ uint64_t sm[kSortCap];
    __shared__ uint32_t sh[kDigitBins];
    __shared__ uint32_t scan_buf[kBatchSelectThreads];
    __shared__ uint32_t tl[kTileListCap];
    __shared__ uint32_t s_vals[4];
    const int seg = blockIdx.y;
    const int t = threadIdx.x;
    const int lane = lane_id();
    const uint32_t *row = rows + (int64_t)seg * ld;
    const uint32_t *tm = tmax + (int64_t)seg * tld;
    const int64_t tiles = (n + 31) / 32;
    TileKeys keys;
    keys.load(tm, tiles);

    // 1. the bound (tile_max_bound)
    const uint32_t bound = tile_max_bound(keys, o.k, sh, scan_buf, s_vals);

    // 2. tiles reaching the bound, then their elements >= bound
    if (t == 0) {
        s_vals[2] = 0u;  // listed tiles
        s_vals[3] = 0u;  // kept ranks
    }
    __syncthreads();
    keys.for_each([&](int64_t i, bool ok, uint32_t key) {
        const bool take = ok && key >= bound;
        const uint64_t m = __ballot(take);
        if (m == 0) return;
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&s_vals[2], (uint32_t)__popcll(m));
        base = (uint32_t)__shfl(base, 0);
        const uint32_t pos = base + (uint32_t)lanes_below(m);
        if (take && pos < (uint32_t)kTileListCap) tl[pos] = (uint32_t)i;
    });
    __syncthreads();
    const uint32_t listed = s_vals[2];
    bool overflow = listed > (uint32_t)kTileListCap;
    if (!overflow) {
        // half-wave h takes listed tiles h, h + 32, ...; lane l of it element
        // l.  Sixteen tiles' loads are issued before any is used, and each
        // wave reserves its kept slots with one LDS atomic per round.
        constexpr int kGatherUnroll = 16;
        const int half = t >> 5;
        const int l = t & 31;
        const int halves = blockDim.x >> 5;
        for (uint32_t j0 = 0; j0 < listed; j0 += (uint32_t)(halves * kGatherUnroll)) {
            uint32_t key[kGatherUnroll];
            int64_t e[kGatherUnroll];
#pragma unroll
            for (int u = 0; u < kGatherUnroll; ++u) {
                const uint32_t j = j0 + (uint32_t)(u * halves + half);
                e[u] = (j < listed) ? (int64_t)tl[j < (uint32_t)kTileListCap ? j : 0u] * 32 + l : n;
                key[u] = row[e[u] < n ? e[u] : n - 1];  // unconditional load (see scan_tiles)
            }
#pragma unroll
            for (int u = 0; u < kGatherUnroll; ++u) key[u] = row_key(key[u]);
            uint64_t mk[kGatherUnroll];
            uint32_t total = 0;
#pragma unroll
            for (int u = 0; u < kGatherUnroll; ++u) {
                mk[u] = __ballot(e[u] < n && key[u] >= bound);
                total += (uint32_t)__popcll(mk[u]);
            }
            if (total == 0) continue;
            uint32_t base = 0;
            if (lane == 0) base = atomicAdd(&s_vals[3], total);
            base = (uint32_t)__shfl(base, 0);
#pragma unroll
            for (int u = 0; u < kGatherUnroll; ++u) {
                const uint32_t pos = base + (uint32_t)lanes_below(mk[u]);
                if (((mk[u] >> lane) & 1ull) && pos < (uint32_t)kSortCap)
                    sm[pos] = make_rank(key[u], (uint32_t)e[u]);
                base += (uint32_t)__popcll(mk[u]);
            }
        }
        __syncthreads();
        overflow = s_vals[3] > (uint32_t)kSortCap;
    }
    if (overflow) {
        __syncthreads();
        select_row_exactly(row, n, o, seg, sm, sh, scan_buf, s_vals);
        return;
    }

    // 3. sort what was kept (at least k ranks) and write the best k
    const int kept = (int)s_vals[3];
    int msz = 64;
    while (msz < kept) msz <<= 1;
    for (int i = kept + t; i < msz; i += blockDim.x) sm[i] = 0ull;
    __syncthreads();
    block_sort_desc(sm, msz);
    for (int r = t; r < o.k; r += blockDim.x) write_result(o, seg, r, sm[r]);
}

// Per query, the threshold of the batched filtered search (mfma_filter.hip):
// thr[seg] = the value of tile_max_bound over that query's per-tile maxima of
// the rows' lower bounds.  At least k tiles reach it and each holds a row whose
// lower bound, hence whose fp32 score, reaches it, so the k-th largest score
// is at or above it; -inf when there are fewer than k tiles (every row stays a
// candidate).
__global__ __launch_bounds__(kBatchSelectThreads) void tile_threshold_kernel(const uint32_t *__restrict__ tmax,
                                                                           int64_t tld, int64_t tiles, int k,
                                                                           float *__restrict__ thr) {
    __shared__ uint32_t sh[kDigitBins];
    __shared__ uint32_t scan_buf[kBatchSelectThreads];
    __shared__ uint32_t s_vals[4];
    const int seg = blockIdx.x;
    TileKeys keys;
    keys.load(tmax + (int64_t)seg * tld, tiles);
    const uint32_t bound = tile_max_bound(keys, k, sh, scan_buf, s_vals);
    // keys below -inf's stand for nothing real: every row is a candidate then
    if (threadIdx.x == 0)
        thr[seg] = (bound > order_key_f32(-INFINITY)) ? f32_of_order_key(bound) : -INFINITY;
}

hipError_t launch_tile_threshold(const float *tmax, int64_t tld, int64_t n, int segments, int k, float *thr,
                                 hipStream_t stream) {
    const int64_t tiles = (n + 31) / 32;
    hipLaunchKernelGGL(tile_threshold_kernel, dim3((unsigned)segments), dim3(kBatchSelectThreads), 0, stream,
                       reinterpret_cast<const uint32_t *>(tmax), tld, tiles, k, thr);
    return hipGetLastError();
}

// ---------------------------------------------------------------- candidate lists

// Per segment (one workgroup each), the best k of the candidate lists that
// launch_filtered_collect left in the slices of its waves: at least k ranks in
// all (the threshold that admitted them certifies k rows).  Up to kSortCap
// ranks are sorted in LDS.  More (many equal scores at the threshold) first
// pin the k-th largest rank with eight histogram passes of 8 bits over the
// slices in memory -- ranks are distinct, so exactly k are at or above it --
// and sort those.  The slices are read in place: with up to kFlatSlices of
// them their offsets go through LDS and each thread loads its candidates
// independently; otherwise each wave walks whole slices.
// Up to this many slices (waves of the collect pass per segment) the slices'
// offsets go through LDS and every candidate is read by one independent load
// (for_each_candidate_flat); more slices are walked one at a time by each wave.
constexpr int kFlatSlices = kBatchSelectThreads;

// Candidate i of a segment lies in the last slice w with off[w] <= i (off: the
// exclusive prefix sums of the slices' counts, off[waves] = m), at position
// i - off[w] of it.  Eight candidates per thread are located and loaded
// before any is used.
template <class F>
__device__ __forceinline__ void for_each_candidate_flat(const uint64_t *__restrict__ c, const uint32_t *off,
                                                        int waves, int64_t rows_per_wave, uint32_t m, F f) {
    constexpr int U = 8;
    for (uint32_t i0 = 0; i0 < m; i0 += (uint32_t)(U * kBatchSelectThreads)) {
        uint64_t r[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t i = i0 + (uint32_t)(u * kBatchSelectThreads) + threadIdx.x;
            ok[u] = i < m;
            int lo = 0, hi = waves;  // off[lo] <= i < off[hi] while i < m
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (off[mid] <= i) lo = mid; else hi = mid;
            }
            r[u] = c[ok[u] ? (int64_t)lo * rows_per_wave + (i - off[lo]) : 0];
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (ok[u]) f(r[u]);
    }
}

template <class F>
__device__ __forceinline__ void for_each_candidate(const uint64_t *__restrict__ c, const uint32_t *__restrict__ cn,
                                                   int waves, int64_t rows_per_wave, F f) {
    constexpr int kWaves = kBatchSelectThreads / 64;
    const int lane = threadIdx.x & 63;
    for (int w = threadIdx.x >> 6; w < waves; w += kWaves) {
        const int64_t cw = (int64_t)cn[w] < rows_per_wave ? (int64_t)cn[w] : rows_per_wave;
        const uint64_t *__restrict__ cs = c + (int64_t)w * rows_per_wave;
        for (int64_t i = lane; i < cw; i += 64) f(cs[i]);
    }
}

__global__ __launch_bounds__(kBatchSelectThreads) void candidate_select_kernel(
    const uint64_t *__restrict__ cand, int64_t ld, const uint32_t *__restrict__ cnt, int64_t cnt_ld, int waves,
    int64_t rows_per_wave, SelectOut o) {
    __shared__ uint64_t sm[kSortCap];
    __shared__ uint32_t hist[256];
    __shared__ uint64_t s_prefix;
    __shared__ int s_need;
    __shared__ uint32_t s_kept;
    __shared__ uint32_t s_m;
    __shared__ uint32_t off[kFlatSlices + 1];
    __shared__ uint32_t scan_buf[kBatchSelectThreads];
    const int seg = blockIdx.x;
    const int t = threadIdx.x;
    const int k = o.k;
    const uint64_t *__restrict__ c = cand + (int64_t)seg * ld;
    const uint32_t *__restrict__ cn = cnt + (int64_t)seg * cnt_ld;
    const bool flat = waves <= kFlatSlices;  // uniform
    if (t == 0) {
        s_m = 0u;
        s_kept = 0u;
    }
    __syncthreads();
    if (flat) {
        const uint32_t v = t < waves ? (uint32_t)min((int64_t)cn[t], rows_per_wave) : 0u;
        const uint32_t incl = block_inclusive_scan(v, scan_buf);
        if (t < waves) off[t] = incl - v;
        if (t == waves - 1) {
            off[waves] = incl;
            s_m = incl;
        }
    } else {
        uint32_t part = 0u;
        for (int w = t; w < waves; w += kBatchSelectThreads) part += min((int64_t)cn[w], rows_per_wave);
        if (part) atomicAdd(&s_m, part);
    }
    __syncthreads();
    const uint32_t m = s_m;
    auto walk = [&](auto f) {
        if (flat)
            for_each_candidate_flat(c, off, waves, rows_per_wave, m, f);
        else
            for_each_candidate(c, cn, waves, rows_per_wave, f);
    };
    uint64_t kth = 0ull;  // keep ranks >= kth
    if (m > (uint32_t)kSortCap) {
        uint64_t prefix = 0ull, mask = 0ull;
        int need = k;
        for (int shift = 56; shift >= 0; shift -= 8) {
            for (int b = t; b < 256; b += kBatchSelectThreads) hist[b] = 0u;
            __syncthreads();
            walk([&](uint64_t r) {
                if ((r & mask) == prefix) atomicAdd(&hist[(r >> shift) & 255u], 1u);
            });
            __syncthreads();
            if (t == 0) {  // the bin, from the top, in which the need-th largest lies
                int above = 0, b = 255;
                for (; b > 0 && above + (int)hist[b] < need; --b) above += (int)hist[b];
                s_need = need - above;
                s_prefix = prefix | ((uint64_t)b << shift);
            }
            __syncthreads();
            need = s_need;
            prefix = s_prefix;
            mask |= 255ull << shift;
            __syncthreads();
        }
        kth = prefix;  // the k-th largest rank itself
    }
    walk([&](uint64_t r) {
        if (r >= kth) {
            const uint32_t pos = atomicAdd(&s_kept, 1u);
            if (pos < (uint32_t)kSortCap) sm[pos] = r;
        }
    });
    __syncthreads();
    const int kept = (int)min(s_kept, (uint32_t)kSortCap);  // m <= kSortCap, or exactly k
    int M = 64;
    while (M < kept) M <<= 1;
    for (int i = kept + t; i < M; i += kBatchSelectThreads) sm[i] = 0ull;
    __syncthreads();
    block_sort_desc(sm, M);
    for (int r = t; r < k; r += kBatchSelectThreads) write_result(o, seg, r, sm[r]);
}

hipError_t launch_candidate_select(const uint64_t *cand, int64_t ld, const uint32_t *cnt, int64_t cnt_ld,
                                   int waves, int64_t rows_per_wave, int segments, int k, int32_t *out_idx,
                                   float *out_scores, hipStream_t stream) {
    if (k < 1 || k > kSortCap || waves < 1 || waves > cnt_ld || rows_per_wave < 1 || rows_per_wave > ld)
        return hipErrorInvalidValue;
    SelectOut o;
    o.k = k;
    o.out_idx = out_idx;
    o.out_val = reinterpret_cast<uint32_t *>(out_scores);
    hipLaunchKernelGGL(candidate_select_kernel, dim3(segments), dim3(kBatchSelectThreads), 0, stream, cand, ld, cnt,
                       cnt_ld, waves, rows_per_wave, o);
    return hipGetLastError();
}

hipError_t launch_tile_bound_select(const float *rows, int64_t ld, int64_t n, const float *tmax, int64_t tld,
                                    int segments, int k, int32_t *out_idx, float *out_scores, hipStream_t stream) {
    SelectOut o;
    o.k = k;
    o.out_idx = out_idx;
    o.out_val = reinterpret_cast<uint32_t *>(out_scores);
    hipLaunchKernelGGL(tile_bound_select_kernel, dim3(1, segments), dim3(kBatchSelectThreads), 0, stream,
                       reinterpret_cast<const uint32_t *>(rows), ld, n, reinterpret_cast<const uint32_t *>(tmax),
                       tld, o);
    return hipGetLastError();
}

}  // namespace rt
