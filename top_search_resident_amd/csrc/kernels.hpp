// kernels.hpp -- host-side launchers of the gfx950 kernels (internal to
// libresident_topk; the public C ABI is include/resident_topk.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rt {

// Workgroup shape of the streaming kernels: 4 waves of 64 lanes.
constexpr int kStreamWaves = 4;
constexpr int kStreamThreads = kStreamWaves * 64;
// Merge workgroups hold up to this many ranks in LDS (64 KiB).
constexpr int kMergeEntries = 8192;
constexpr int kMergeThreads = 1024;
// Batched scoring: one 512-thread workgroup per CU, 32 queries x 64 rows per wave tile.
constexpr int kMfmaThreads = 512;
constexpr int kMfmaMaxQ = 32;
constexpr int kMfmaMaxD = 1024;

// Fast inner-product path: d % 4 == 0 and d / 4 <= 64 * 8.
bool gemv_fast_path_ok(int d);

// Streaming scorer + per-wave selection; grid (wgs_per_seg, segments).
hipError_t launch_gemv_topk(const float *corpus, int64_t n, int d, const float *queries, int segments,
                            int k, int kp, int64_t rows_per_wave, int wgs_per_seg,
                            uint64_t *wg_lists, uint64_t *seg_thr, hipStream_t stream);

// Streaming selection over raw 32-bit arrays; dtype 0 = int32, 1 = fp32.
hipError_t launch_select_topk(const void *base, int64_t seg_stride, int64_t n, int dtype, int segments,
                              int k, int kp, int64_t groups_per_wave, int wgs_per_seg,
                              uint64_t *wg_lists, uint64_t *seg_thr, hipStream_t stream);

// One level of the tree merge: every workgroup merges `fan_in` lists into one.
// mode 0: write the merged lists to out_lists; mode 1: search outputs (index +
// fp32 score from the rank); mode 2: select outputs (index + the source's
// 32-bit element).  Modes 1 and 2 also reset seg_thr.
hipError_t launch_merge(const uint64_t *in_lists, int lists_per_seg, int fan_in, int segments, int kp,
                        uint64_t *out_lists, int mode, int k, int32_t *out_idx, void *out_val,
                        const void *src, int64_t src_seg_stride, uint64_t *seg_thr, hipStream_t stream);

hipError_t launch_reset(uint64_t *seg_thr, int count, hipStream_t stream);

// Batched inner products S[q][row] (row stride ld) on MFMA; q <= 32, d % 4 == 0, d <= 1024.
hipError_t prepare_mfma_scores();
hipError_t launch_mfma_scores(const float *corpus, int64_t n, int d, const float *queries, int q,
                              float *scores, int64_t ld, int num_cus, hipStream_t stream);

}  // namespace rt
