// engine.hip -- the C ABI of libresident_topk (declared in include/resident_topk.h).
//
// "GPU-Resident Top-K for Agentic RAG" (A. Banerjee): an engine allocates every
// device buffer once at initialisation, sized for the worst case (section 3,
// "Problem C"; section 4, Step 0), the corpus is uploaded once and stays
// resident (Step 1), and each search is scoring + per-block top-K + merge on the
// device (Steps 2-5).  This file owns the buffers, validates arguments on the
// host before anything is enqueued, plans the launch shapes and enqueues the
// kernels of stream_topk.hip, mfma_scores.hip and merge_topk.hip.
#include <hip/hip_runtime.h>

#include <new>

#include "../../include/resident_topk.h"
#include "kernels.hpp"

namespace {

constexpr int64_t kMaxN = 2147483647LL;
constexpr int32_t kMaxD = 65536;
constexpr int32_t kMaxK = 1024;
constexpr int32_t kMaxQ = 32;
// Per-workgroup list storage (ranks) for each of the two ping-pong buffers.
constexpr int64_t kListEntries = int64_t(1) << 22;
// Most waves the streaming stage uses per segment.
constexpr int64_t kMaxWavesPerSeg = 4096;

int kp_for(int k) {
    int kp = 64;
    while (kp < k) kp <<= 1;
    return kp;
}

struct Plan {
    int wgs;            // workgroups per segment in the streaming stage
    int64_t per_wave;   // rows (scoring) or 16-byte groups (raw arrays) per wave
};

// Split `units` (rows or 16-byte groups) of each of `segments` segments over
// waves: at least `min_per_wave` units per wave, at most kMaxWavesPerSeg waves
// per segment, and the per-workgroup lists must fit one ping-pong buffer.
Plan plan_stream(int64_t units, int segments, int kp, int64_t min_per_wave) {
    int64_t waves = (units + min_per_wave - 1) / min_per_wave;
    if (waves > kMaxWavesPerSeg) waves = kMaxWavesPerSeg;
    if (waves < 1) waves = 1;
    int64_t wgs = (waves + rt::kStreamWaves - 1) / rt::kStreamWaves;
    const int64_t cap = kListEntries / ((int64_t)segments * kp);
    if (wgs > cap) wgs = cap;
    if (wgs < 1) wgs = 1;
    waves = wgs * rt::kStreamWaves;
    Plan p;
    p.wgs = (int)wgs;
    p.per_wave = (units + waves - 1) / waves;
    if (p.per_wave < 1) p.per_wave = 1;
    return p;
}

}  // namespace

struct rt_engine {
    int device = 0;
    int num_cus = 0;
    int64_t max_n = 0;
    int32_t max_d = 0, max_k = 0, max_q = 0;
    int64_t resident_n = 0;
    int32_t resident_d = 0;
    float *corpus = nullptr;
    float *scores = nullptr;  // batched scores, max_q x roundup(max_n, 64); only when max_q > 1
    uint64_t *lists[2] = {nullptr, nullptr};
    uint64_t *seg_thr = nullptr;
    hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
    bool profiling = false;
    bool had_batch_kernel = false;
    bool dirty = false;
    int32_t last_hip = 0;
};

static rt_status hip_fail(rt_engine *e, hipError_t err) {
    if (e) {
        e->last_hip = (int32_t)err;
        e->dirty = true;
    }
    (void)hipGetLastError();
    return RT_EHIP;
}

extern "C" {

const char *rt_status_string(rt_status s) {
    switch (s) {
        case RT_OK: return "ok";
        case RT_EINVAL: return "invalid argument";
        case RT_ESTATE: return "invalid state (no corpus resident, or dimension mismatch)";
        case RT_ENOMEM: return "device memory allocation failed";
        case RT_EHIP: return "HIP runtime error";
    }
    return "unknown status";
}

rt_status rt_check_create(int64_t max_n, int32_t max_d, int32_t max_k, int32_t max_q) {
    if (max_n < 1 || max_n > kMaxN) return RT_EINVAL;
    if (max_d < 1 || max_d > kMaxD) return RT_EINVAL;
    if (max_k < 1 || max_k > kMaxK) return RT_EINVAL;
    if (max_q < 1 || max_q > kMaxQ) return RT_EINVAL;
    return RT_OK;
}

rt_status rt_check_upload(int64_t max_n, int32_t max_d, const void *corpus, int64_t n, int32_t d) {
    if (corpus == nullptr) return RT_EINVAL;
    if (n < 1 || n > max_n) return RT_EINVAL;
    if (d < 1 || d > max_d) return RT_EINVAL;
    return RT_OK;
}

rt_status rt_check_search(int32_t max_k, int32_t max_q, int64_t resident_n, const void *queries, int32_t q,
                          int32_t k, const void *out_idx, const void *out_scores) {
    if (queries == nullptr || out_idx == nullptr || out_scores == nullptr) return RT_EINVAL;
    if (q < 1 || q > max_q) return RT_EINVAL;
    if (k < 1 || k > max_k) return RT_EINVAL;
    if (resident_n < 1) return RT_ESTATE;
    if (k > resident_n) return RT_EINVAL;
    return RT_OK;
}

rt_status rt_check_select(int32_t max_k, const void *values, int32_t dtype, int64_t n, int32_t k,
                          const void *out_idx, const void *out_values) {
    if (values == nullptr || out_idx == nullptr || out_values == nullptr) return RT_EINVAL;
    if (dtype != RT_DTYPE_INT32 && dtype != RT_DTYPE_FLOAT32) return RT_EINVAL;
    if ((reinterpret_cast<uintptr_t>(values) & 3u) != 0) return RT_EINVAL;
    if (n < 1 || n > kMaxN) return RT_EINVAL;
    if (k < 1 || k > max_k || k > n) return RT_EINVAL;
    return RT_OK;
}

void rt_engine_destroy(rt_engine *e) {
    if (!e) return;
    int prev = 0;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(e->device);
    (void)hipDeviceSynchronize();
    (void)hipFree(e->corpus);
    (void)hipFree(e->scores);
    (void)hipFree(e->lists[0]);
    (void)hipFree(e->lists[1]);
    (void)hipFree(e->seg_thr);
    for (auto &ev : e->ev)
        if (ev) (void)hipEventDestroy(ev);
    (void)hipSetDevice(prev);
    delete e;
}

rt_status rt_engine_create(int64_t max_n, int32_t max_d, int32_t max_k, int32_t max_q, int32_t device,
                           rt_engine **out) {
    if (out == nullptr) return RT_EINVAL;
    *out = nullptr;
    rt_status st = rt_check_create(max_n, max_d, max_k, max_q);
    if (st != RT_OK) return st;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev) {
        (void)hipGetLastError();
        return device < 0 ? RT_EINVAL : RT_EHIP;
    }
    rt_engine *e = new (std::nothrow) rt_engine();
    if (!e) return RT_ENOMEM;
    e->device = device;
    e->max_n = max_n;
    e->max_d = max_d;
    e->max_k = max_k;
    e->max_q = max_q;
    int prev = 0;
    (void)hipGetDevice(&prev);
    hipError_t err = hipSetDevice(device);
    if (err != hipSuccess) {
        delete e;
        return hip_fail(nullptr, err);
    }
    err = hipDeviceGetAttribute(&e->num_cus, hipDeviceAttributeMultiprocessorCount, device);
    if (err != hipSuccess || e->num_cus < 1) e->num_cus = 256;

    auto alloc = [&](void **p, size_t bytes) -> bool {
        if (hipMalloc(p, bytes) != hipSuccess) {
            (void)hipGetLastError();
            return false;
        }
        return true;
    };
    const int64_t ld = (max_n + 63) / 64 * 64;
    bool ok = alloc(reinterpret_cast<void **>(&e->corpus), sizeof(float) * (size_t)max_n * (size_t)max_d) &&
              alloc(reinterpret_cast<void **>(&e->lists[0]), sizeof(uint64_t) * (size_t)kListEntries) &&
              alloc(reinterpret_cast<void **>(&e->lists[1]), sizeof(uint64_t) * (size_t)kListEntries) &&
              alloc(reinterpret_cast<void **>(&e->seg_thr), sizeof(uint64_t) * (size_t)kMaxQ);
    if (ok && max_q > 1) ok = alloc(reinterpret_cast<void **>(&e->scores), sizeof(float) * (size_t)max_q * (size_t)ld);
    if (!ok) {
        rt_engine_destroy(e);
        (void)hipSetDevice(prev);
        return RT_ENOMEM;
    }
    err = hipMemset(e->seg_thr, 0, sizeof(uint64_t) * kMaxQ);
    if (err == hipSuccess) err = rt::prepare_mfma_scores();
    for (int i = 0; i < 4 && err == hipSuccess; ++i) err = hipEventCreate(&e->ev[i]);
    if (err == hipSuccess) err = hipDeviceSynchronize();
    (void)hipSetDevice(prev);
    if (err != hipSuccess) {
        rt_engine_destroy(e);
        (void)hipGetLastError();
        return RT_EHIP;
    }
    *out = e;
    return RT_OK;
}

rt_status upload_corpus_rowmajor(rt_engine *e, const float *corpus, int64_t n, int32_t d) {
    if (!e) return RT_EINVAL;
    rt_status st = rt_check_upload(e->max_n, e->max_d, corpus, n, d);
    if (st != RT_OK) return st;
    int prev = 0;
    (void)hipGetDevice(&prev);
    hipError_t err = hipSetDevice(e->device);
    if (err == hipSuccess)
        err = hipMemcpy(e->corpus, corpus, sizeof(float) * (size_t)n * (size_t)d, hipMemcpyDefault);
    (void)hipSetDevice(prev);
    if (err != hipSuccess) {
        e->resident_n = 0;
        e->resident_d = 0;
        return hip_fail(e, err);
    }
    e->resident_n = n;
    e->resident_d = d;
    return RT_OK;
}

// Enqueue the merge levels for `segments` segments of `lists` per-workgroup lists
// held in e->lists[0]; the last level writes the outputs.
static hipError_t enqueue_merges(rt_engine *e, int lists, int segments, int kp, int mode, int k, int32_t *out_idx,
                                 void *out_val, const void *src, int64_t src_stride, hipStream_t s) {
    const int max_fan = rt::kMergeEntries / kp;
    int cur = 0;
    hipError_t err = hipSuccess;
    while (true) {
        int fan = 1;
        while (fan < lists && fan < max_fan) fan <<= 1;
        const int groups = (lists + fan - 1) / fan;
        const bool last = groups == 1;
        err = rt::launch_merge(e->lists[cur], lists, fan, segments, kp, e->lists[cur ^ 1], last ? mode : 0, k,
                               out_idx, out_val, src, src_stride, e->seg_thr, s);
        if (err != hipSuccess || last) break;
        lists = groups;
        cur ^= 1;
    }
    return err;
}

static hipError_t prologue(rt_engine *e, hipStream_t s) {
    hipError_t err = hipSuccess;
    if (e->dirty) {
        err = rt::launch_reset(e->seg_thr, kMaxQ, s);
        if (err != hipSuccess) return err;
        e->dirty = false;
    }
    if (e->profiling) err = hipEventRecord(e->ev[0], s);
    return err;
}

rt_status search_resident(rt_engine *e, const float *queries, int32_t q, int32_t k, int32_t *out_idx,
                          float *out_scores, void *stream) {
    if (!e) return RT_EINVAL;
    rt_status st = rt_check_search(e->max_k, e->max_q, e->resident_n, queries, q, k, out_idx, out_scores);
    if (st != RT_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int prev = 0;
    (void)hipGetDevice(&prev);
    hipError_t err = hipSetDevice(e->device);
    const int64_t n = e->resident_n;
    const int d = e->resident_d;
    const int kp = kp_for(k);
    const bool batched = q > 1 && e->scores != nullptr && d % 4 == 0 && d <= rt::kMfmaMaxD;
    e->had_batch_kernel = batched;
    if (err == hipSuccess) err = prologue(e, s);
    int wgs = 0;
    if (err == hipSuccess && batched) {
        const int64_t ld = (n + 63) / 64 * 64;
        err = rt::launch_mfma_scores(e->corpus, n, d, queries, q, e->scores, ld, e->num_cus, s);
        if (err == hipSuccess && e->profiling) err = hipEventRecord(e->ev[3], s);
        // each wave streams at least 1024 scores (256 groups of 4)
        const Plan p = plan_stream((n + 3) / 4, q, kp, 256);
        wgs = p.wgs;
        if (err == hipSuccess)
            err = rt::launch_select_topk(e->scores, ld, n, 1, q, k, kp, p.per_wave, p.wgs, e->lists[0], e->seg_thr, s);
    } else if (err == hipSuccess) {
        const Plan p = plan_stream(n, q, kp, 32);
        wgs = p.wgs;
        err = rt::launch_gemv_topk(e->corpus, n, d, queries, q, k, kp, p.per_wave, p.wgs, e->lists[0], e->seg_thr, s);
    }
    if (err == hipSuccess && e->profiling) err = hipEventRecord(e->ev[1], s);
    if (err == hipSuccess) err = enqueue_merges(e, wgs, q, kp, 1, k, out_idx, out_scores, nullptr, 0, s);
    if (err == hipSuccess && e->profiling) err = hipEventRecord(e->ev[2], s);
    (void)hipSetDevice(prev);
    if (err != hipSuccess) return hip_fail(e, err);
    return RT_OK;
}

rt_status topk_select(rt_engine *e, const void *values, int32_t dtype, int64_t n, int32_t k, int32_t *out_idx,
                      void *out_values, void *stream) {
    if (!e) return RT_EINVAL;
    rt_status st = rt_check_select(e->max_k, values, dtype, n, k, out_idx, out_values);
    if (st != RT_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int prev = 0;
    (void)hipGetDevice(&prev);
    hipError_t err = hipSetDevice(e->device);
    const int kp = kp_for(k);
    e->had_batch_kernel = false;
    if (err == hipSuccess) err = prologue(e, s);
    const int64_t head = (int64_t)((reinterpret_cast<uintptr_t>(values) & 15u) >> 2);
    const Plan p = plan_stream((n + head + 3) / 4, 1, kp, 256);
    if (err == hipSuccess)
        err = rt::launch_select_topk(values, 0, n, dtype, 1, k, kp, p.per_wave, p.wgs, e->lists[0], e->seg_thr, s);
    if (err == hipSuccess && e->profiling) err = hipEventRecord(e->ev[1], s);
    if (err == hipSuccess) err = enqueue_merges(e, p.wgs, 1, kp, 2, k, out_idx, out_values, values, 0, s);
    if (err == hipSuccess && e->profiling) err = hipEventRecord(e->ev[2], s);
    (void)hipSetDevice(prev);
    if (err != hipSuccess) return hip_fail(e, err);
    return RT_OK;
}

int32_t rt_last_hip_error(const rt_engine *e) { return e ? e->last_hip : 0; }

rt_status rt_profile_enable(rt_engine *e, int32_t on) {
    if (!e) return RT_EINVAL;
    e->profiling = on != 0;
    return RT_OK;
}

rt_status rt_profile_read(rt_engine *e, float *ms3) {
    if (!e || !ms3) return RT_EINVAL;
    ms3[0] = ms3[1] = ms3[2] = 0.f;
    hipError_t err = hipEventElapsedTime(&ms3[0], e->ev[0], e->ev[1]);
    if (err == hipSuccess) err = hipEventElapsedTime(&ms3[1], e->ev[1], e->ev[2]);
    if (err == hipSuccess && e->had_batch_kernel) err = hipEventElapsedTime(&ms3[2], e->ev[0], e->ev[3]);
    if (err != hipSuccess) {
        e->last_hip = (int32_t)err;
        (void)hipGetLastError();
        return RT_EHIP;
    }
    return RT_OK;
}

rt_status rt_engine_info(const rt_engine *e, int64_t *out7) {
    if (!e || !out7) return RT_EINVAL;
    out7[0] = e->max_n;
    out7[1] = e->max_d;
    out7[2] = e->max_k;
    out7[3] = e->max_q;
    out7[4] = e->resident_n;
    out7[5] = e->resident_d;
    out7[6] = e->device;
    return RT_OK;
}

}  // extern "C"
