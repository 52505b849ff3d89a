// kernels.hpp -- host-side launchers of the gfx950 kernels (internal to
// libresident_topk; the public C ABI is include/resident_topk.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rt {

// Workgroup shape of the scoring kernels: kGemvWaves waves of 64 lanes for
// lists of up to 256 entries (a merge-tree node merges its lists with all the
// workgroup's waves), 4 waves for longer lists (all wave lists must fit the
// merge LDS).
constexpr int kGemvWaves = 8;
// Rows per wave up to which the scorer loads two steps ahead (below, every
// step of a short range would pay a full memory latency; above, the chip is
// bandwidth-bound and lookahead only adds outstanding requests).
constexpr int64_t kGemvLookaheadRows = 128;
constexpr int gemv_waves(int kp) { return kp <= 256 ? kGemvWaves : 4; }
// Raw-array selection runs 16-wave workgroups that share a certified bound in
// LDS (all 16 lists must fit the merge LDS, so only for lists <= 256 entries).
constexpr int select_waves(int kp) { return kp <= 256 ? 16 : 4; }
// LDS ranks a workgroup uses to merge lists in the merge tree (32 KiB); a tree
// node merges kTreeEntries / tree_stride(k, Kp) lists.
constexpr int kTreeEntries = 4096;
// Batched scoring: one workgroup per CU (512 threads for a runtime depth, 1024 for
// the compile-time depths), 32 queries x 32 rows per wave tile.
constexpr int kMfmaThreads = 512;
constexpr int kMfmaMaxQ = 32;
constexpr int kMfmaMaxD = 1024;

// Where the streaming kernels keep the merge tree and where the answer goes.
struct TreeLaunch {
    uint64_t *tree;            // list storage, seg_tree_stride ranks per segment
    uint32_t *counters;        // arrival counters, seg_ctr_stride per segment, all zero between calls
    int64_t seg_tree_stride;   // >= 2 * workgroups_per_segment * kp
    int seg_ctr_stride;        // >= workgroups_per_segment
    int kp;                    // list length: power of two in [64, 1024], >= k
    int k;
    int mode;                  // 1: search (index + fp32 score); 2: select (index + source element);
                               // 3: only the k-th entry's fp32 value (to out_val[segment])
    int32_t *out_idx;          // [segments][k]
    void *out_val;             // [segments][k] 32-bit values
    const void *src;           // mode 2: the selected-from array
    int64_t src_seg_stride;    // mode 2: elements between segments of src
};

// The bf16-filtered exact search (filter_topk.hpp): bound factor and scratch.
struct FilterLaunch {
    float cb;        // e_i = cb |q| |x_i| + delta bounds |bf16 score - fp32 score|
    float delta;
    float *ubuf;     // [segments][uld] upper bounds, written by pass 1
    int64_t uld;
    float *thr;      // [segments] k-th largest lower bound, written by pass 1
    const float *crn = nullptr;  // cosine metric: the rows' L2 norms (null: inner product)
    const uint16_t *ub16 = nullptr;  // pass 2: read 16-bit upper bounds (top halves of fp32) from here instead
    bool bounds16 = false;  // single-query passes: pass 1 writes 16-bit bounds at ubuf, pass 2 reads them there
    int ub_tq = 0;          // with ub16: nonzero if tile-major with this many queries per tile (launch_mfma_bound)
    uint64_t *cand = nullptr;     // pass 2 collect mode: candidate ranks (see launch_filtered_collect)
    int64_t cand_ld = 0;
    uint32_t *cand_cnt = nullptr;
    int64_t cnt_ld = 0;
};

// Bound factor cb for depth d (fp64 on the host, rounded up; see filter_topk.hpp)
// and the absolute slack delta (times max(|q|, 1)) for underflow.
float filter_bound_factor(int d);
float filter_underflow_slack(int d);
// Depths the filtered search handles: d % 8 == 0 and the fp32 fast-path shapes.
bool filtered_search_ok(int d);
// Lane-group shape (G = 2^log2g lanes, L 16-byte loads per lane) for rows of
// `blocks` 16-byte blocks (blocks <= 512).
void pick_gemv_shape(int blocks, int *log2g, int *L);

// Exact top-k by inner product for `segments` queries through the bf16 copy
// (pass 1: bounds and the threshold) and the fp32 rows that reach it (pass 2).
// d % 8 == 0.  Grids (wgs1 or wgs2, segments).  `between` (may be null) is
// recorded on the stream after pass 1.
hipError_t launch_filtered_search(const float *corpus, const uint16_t *corpus16, const float *rnorm, int64_t n,
                                  int d, const float *queries, int segments, int64_t rows_per_wave1, int wgs1,
                                  const TreeLaunch &t1, int64_t rows_per_wave2, int wgs2, const TreeLaunch &t2,
                                  const FilterLaunch &f, hipEvent_t between, hipStream_t stream);

// Pass 2 of the filtered search alone: for each of `segments` queries, re-score
// in fp32 the rows whose upper bound f.ubuf[seg][row] reaches f.thr[seg] and
// select among them (grid (wgs, segments)).
hipError_t launch_filtered_pass2(const float *corpus, int64_t n, int d, const float *queries, int segments,
                                 int64_t rows_per_wave, int wgs, const TreeLaunch &t, const FilterLaunch &f,
                                 hipStream_t stream);

// Batched filtered search (mfma_filter.hip).  Depths with a compile-time
// bf16 MFMA bound kernel (d in {256, 384, 512, 768, 1024}); the bound's
// constants: e = |q| (cr |x - bf16(x)| + cx |x|) + delta max(|q|, 1) max(|x|, 1).
bool mfma_filter_ok(int d);
void filter_bound_constants_batched(int d, float *cr, float *cx, float *delta);
hipError_t prepare_mfma_filter();
// Pass 1 for q <= 32 queries: 16-bit upper bounds (the top halves of fp32
// values rounded toward +inf) at (uint16_t *)ubuf, tile-major: the bound of
// (query j, row r) at (r / 32) * 32 * q + 32 j + r % 32, i.e. q * roundup(n, 32)
// entries, which pass 2 reads through FilterLaunch::ub16 with ub_tq = q; and,
// per query, the largest lower bound of every 32-row tile, tlb[query * tld +
// tile].  rnorm[i] = |x_i|, rerr[i] >= |x_i - bf16(x_i)| (both readable up to
// a multiple of 32 rows past n).
hipError_t launch_mfma_bound(const uint16_t *corpus16, int64_t n, int d, const float *queries, int q,
                             const float *rnorm, const float *rerr, float *ubuf, float *tlb, int64_t tld,
                             int num_cus, hipStream_t stream);
// Per query, thr[seg] <= the k-th largest of that query's tile maxima of lower
// bounds tmax[seg * tld + tile] (a bin edge below it; -inf when n has fewer
// than k tiles), so at least k rows have a lower bound at or above it.
hipError_t launch_tile_threshold(const float *tmax, int64_t tld, int64_t n, int segments, int k, float *thr,
                                 hipStream_t stream);

// Pass 2 of the batched filtered search for large k, in two launches.  Every
// row whose upper bound reaches f.thr[seg] is re-scored in fp32 exactly as in
// launch_filtered_pass2; if its score reaches the threshold too, its rank goes
// to the slice of the list of the wave that took the row: the wave over rows
// [w * rows_per_wave, ..) writes them from f.cand[seg * f.cand_ld + w *
// rows_per_wave] on (f.cand_ld >= n: slices cannot overlap) and their number
// to f.cand_cnt[seg * f.cnt_ld + w], for every w < wgs * collect_waves (so
// f.cnt_ld >= that, and nothing needs clearing between calls).  Then
// candidate_select gathers each segment's slices, sorts them and writes the
// best k (index + score).
constexpr int collect_waves() { return gemv_waves(64); }
hipError_t launch_filtered_collect(const float *corpus, int64_t n, int d, const float *queries, int segments,
                                   int64_t rows_per_wave, int wgs, const TreeLaunch &t, const FilterLaunch &f,
                                   hipStream_t stream);
hipError_t launch_candidate_select(const uint64_t *cand, int64_t ld, const uint32_t *cnt, int64_t cnt_ld,
                                   int waves, int64_t rows_per_wave, int segments, int k, int32_t *out_idx,
                                   float *out_scores, hipStream_t stream);

// err[row] >= the L2 norm of corpus row - its bf16 copy, for rows < n.
hipError_t launch_bf16_row_errors(const float *corpus, int64_t n, int d, float *err, int num_cus,
                                  hipStream_t stream);

// corpus16[i] = bf16 of corpus[i] (round to nearest even), i < count; *bad is set
// to 1 if any value is not finite or rounds to infinity (the caller clears it).
hipError_t launch_to_bf16(const float *corpus, uint16_t *corpus16, int64_t count, uint32_t *bad, int num_cus,
                          hipStream_t stream);

// Entries between consecutive lists in the merge tree for top-k with lists of
// kp entries: the smallest power of two >= k when k <= 32 (only the first k
// entries of a list matter), else kp.  A tree node merges kTreeEntries / stride
// lists.
int tree_stride(int k, int kp);

// Fast inner-product path: d % 4 == 0 and d / 4 <= 64 * 8.
bool gemv_fast_path_ok(int d);

// Fused scoring + selection + merge for `segments` queries; grid (wgs_per_seg, segments).
// rnorm == nullptr: inner product; otherwise cosine, rnorm[i] = |row i|.
hipError_t launch_gemv_topk(const float *corpus, int64_t n, int d, const float *queries, const float *rnorm,
                            int segments, int64_t rows_per_wave, int wgs_per_seg, const TreeLaunch &t,
                            hipStream_t stream);

// rnorm[i] = L2 norm of corpus row i (fp64 sum of squares, rounded to fp32).
hipError_t launch_row_norms(const float *corpus, int64_t n, int d, float *rnorm, int num_cus, hipStream_t stream);

// Selection + merge over `segments` raw 32-bit arrays (dtype 0 = int32, 1 = fp32)
// of n elements, seg_stride elements apart.
hipError_t launch_select_topk(const void *base, int64_t seg_stride, int64_t n, int dtype, int segments,
                              int64_t groups_per_wave, int wgs_per_seg, const TreeLaunch &t, hipStream_t stream);

// Clear merge-tree counters after a failed launch left them in an unknown state.
hipError_t launch_zero_counters(uint32_t *counters, int64_t count, hipStream_t stream);

// Batched inner products S[q][row] (row stride ld) on MFMA; q <= 32, d % 4 == 0, d <= 1024.
// Also writes, per query, the largest score of every 32-row tile:
// tmax[query * tld + tile], tile = row / 32.  rnorm != nullptr selects cosine
// scores (rnorm[i] = |row i|, readable up to a multiple of 4 rows past n).
hipError_t prepare_mfma_scores();
hipError_t launch_mfma_scores(const float *corpus, int64_t n, int d, const float *queries, int q,
                              const float *rnorm, float *scores, int64_t ld, float *tmax, int64_t tld, int num_cus,
                              hipStream_t stream);

// Exact top-k (k <= 1024) of each of `segments` fp32 score rows (ld apart) given
// their 32-element tile maxima (tld apart); writes index + score per row.
hipError_t launch_tile_bound_select(const float *rows, int64_t ld, int64_t n, const float *tmax, int64_t tld,
                                    int segments, int k, int32_t *out_idx, float *out_scores, hipStream_t stream);

}  // namespace rt
