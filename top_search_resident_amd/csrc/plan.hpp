// plan.hpp -- launch planning shared by the entry points (host only).
//
// A streaming launch splits the rows (scoring) or 16-byte groups (raw arrays)
// of each segment over waves; the per-workgroup best-K lists then go up the
// merge tree, whose list storage (tree_ranks ranks) and arrival counters
// (max_wgs per segment) the caller provides.
#pragma once
#include <stdint.h>

#include "kernels.hpp"

namespace rt {

// Streaming waves per CU the planner aims for (measured on MI355X): 8 for the
// scorer -- one 8-wave workgroup per CU beat 4-wave pairs and 16 waves per CU
// from 10k x 384 to 1M x 1024 -- and 16 for raw-array selection (1e8 int32).
constexpr int64_t kScoreWavesPerCu = 8;
constexpr int64_t kSelectWavesPerCu = 16;

// List length for top-k: the smallest power of two >= max(k, 64).
inline int kp_for(int k) {
    int kp = 64;
    while (kp < k) kp <<= 1;
    return kp;
}

struct Plan {
    int wgs;            // workgroups per segment
    int64_t per_wave;   // rows (scoring) or 16-byte groups (raw arrays) per wave
};

// Split `units` of each of `segments` segments over waves: at least
// `min_per_wave` units per wave, about waves_per_cu waves per CU in total, at
// most max_wgs workgroups per segment, and the merge tree (at most 2 * wgs * kp
// ranks per segment) must fit tree_ranks.
inline Plan plan_stream(int64_t units, int segments, int kp, int64_t min_per_wave, int num_cus, int64_t waves_per_cu,
                        int waves_per_wg, int64_t tree_ranks, int64_t max_wgs) {
    int64_t target = (int64_t)num_cus * waves_per_cu / segments;
    if (target < waves_per_wg) target = waves_per_wg;
    int64_t waves = (units + min_per_wave - 1) / min_per_wave;
    if (waves > target) waves = target;
    if (waves < 1) waves = 1;
    int64_t wgs = (waves + waves_per_wg - 1) / waves_per_wg;
    const int64_t cap = tree_ranks / ((int64_t)segments * 2 * kp);
    if (wgs > cap) wgs = cap;
    if (wgs > max_wgs) wgs = max_wgs;
    if (wgs < 1) wgs = 1;
    waves = wgs * waves_per_wg;
    Plan p;
    p.wgs = (int)wgs;
    p.per_wave = (units + waves - 1) / waves;
    if (p.per_wave < 1) p.per_wave = 1;
    return p;
}

// Raw-array selection of n 32-bit values at `values` (4-byte aligned): the
// array is read as the 16-byte groups of its enclosing aligned range.
inline Plan plan_select(const void *values, int64_t n, int kp, int num_cus, int64_t tree_ranks, int64_t max_wgs) {
    const int64_t head = (int64_t)((reinterpret_cast<uintptr_t>(values) & 15u) >> 2);
    return plan_stream((n + head + 3) / 4, 1, kp, 256, num_cus, kSelectWavesPerCu, select_waves(kp), tree_ranks,
                       max_wgs);
}

// Merge-tree description for one launch of `p.wgs` workgroups per segment.
inline TreeLaunch tree_launch(uint64_t *tree, uint32_t *counters, int ctr_stride, const Plan &p, int kp, int k,
                              int mode, int32_t *out_idx, void *out_val, const void *src, int64_t src_stride) {
    TreeLaunch t;
    t.tree = tree;
    t.counters = counters;
    t.seg_tree_stride = 2 * (int64_t)p.wgs * kp;
    t.seg_ctr_stride = ctr_stride;
    t.kp = kp;
    t.k = k;
    t.mode = mode;
    t.out_idx = out_idx;
    t.out_val = out_val;
    t.src = src;
    t.src_seg_stride = src_stride;
    return t;
}

}  // namespace rt
