// engine.hip -- the C ABI of libresident_topk (declared in include/resident_topk.h).
//
// "GPU-Resident Top-K for Agentic RAG" (A. Banerjee): an engine allocates every
// device buffer once at initialisation, sized for the worst case (section 3,
// "Problem C"; section 4, Step 0), the corpus is uploaded once and stays
// resident (Step 1), and each search is scoring + per-block top-K + merge on the
// device (Steps 2-5).  This file owns the buffers, validates arguments on the
// host before anything is enqueued, plans the launch shapes and enqueues the
// kernels of stream_topk.hip and mfma_scores.hip.
#include <hip/hip_runtime.h>

#include <math.h>

#include <atomic>
#include <new>

#include "../../include/resident_topk.h"
#include "cosine_math.hpp"
#include "filter8_host.hpp"
#include "kernels.hpp"
#include "limits.hpp"
#include "plan.hpp"
#include "read_probe.hpp"

namespace {

using rt::kMaxQ;
// Merge-tree list storage (ranks) shared by all segments of a call: 64 MiB.
constexpr int64_t kTreeRanks = int64_t(1) << 23;
// Most streaming workgroups per segment (bounds the counter array).
constexpr int64_t kMaxWgsPerSeg = 2048;
constexpr int64_t kMaxCollectWaves = kMaxWgsPerSeg * rt::collect_waves();

using rt::kp_for;
using rt::kScoreWavesPerCu;
using rt::Plan;

Plan plan_stream(int64_t units, int segments, int kp, int64_t min_per_wave, int num_cus, int64_t waves_per_cu,
                 int waves_per_wg) {
    return rt::plan_stream(units, segments, kp, min_per_wave, num_cus, waves_per_cu, waves_per_wg, kTreeRanks,
                           kMaxWgsPerSeg);
}

// Corpus size (n x d elements) from which a single-query filtered search pays
// off when the engine leaves the choice to the library (RT_FILTER_AUTO), and
// from which it then takes the fp8 first pass.  Below it the plain scan runs:
// the two passes' fixed cost (two launches, two merge trees) outweighs the
// bytes the first pass saves.  Host p50 per query at K = 8, d = 768, MI355X,
// plain / bf16 first pass / fp8 first pass: 20k rows 31.7 / 44.0 / 48.3 us,
// 50k rows 44.4 / 47.9 / 48.9 us, 65k rows 53.1 / 50.6 / 50.2 us, 80k rows
// 56.5 / 54.4 / 51.0 us.  The answer is the same on every path.
constexpr int64_t kFilteredMinElements = int64_t(44) << 20;
constexpr int64_t kFp8MinElements = kFilteredMinElements;

// Waves per CU of the batched filtered search's re-rank (pass 2).  With up to
// 32 queries each gets 1/32 of them, and a wave walks its rows' bounds in
// 512-row chunks, one memory round trip each; twice the scoring kernels' 8
// shortens those chains, while more waves cost more in the merge trees.
// MI355X, 32 x 500k x 768, threshold + re-rank at K = 100 / 1024: 8 waves
// 39.9 / 68.4 us, 12: 37.3 / 65.3, 16: 34.4 / 63.9, 20: 43.5 / 73.2, 32:
// 47.3 / 74.8 us.
constexpr int64_t kBatchRerankWavesPerCu = 16;

// Fewest rows a scoring wave streams: about 24 KB of rows (4 to 32 rows).  A
// small corpus then spreads over more CUs with shorter chains of dependent
// steps per wave (measured on MI355X, p50 per query: 10k x 384 15.8 -> 14.2 us,
// 20k x 768 25.5 -> 20.4 us, 5k x 1024 22.4 -> 14.9 us against a fixed 32 rows);
// large corpora are bound by the waves-per-CU target instead.
int64_t min_rows_per_wave(int d) {
    const int64_t rows = (24576 + 4 * (int64_t)d - 1) / (4 * (int64_t)d);
    return rows < 4 ? 4 : (rows > 32 ? 32 : rows);
}

}  // namespace

// The resident corpus and its row norms.  Engines created with
// rt_engine_create_shared point at the same one; it is freed with the last of
// them.
struct rt_resident {
    std::atomic<int> refs{1};
    int64_t max_n = 0;
    int32_t max_d = 0;
    int64_t n = 0;            // resident rows (0: nothing uploaded)
    int32_t d = 0;
    float *corpus = nullptr;  // max_n x max_d fp32
    float *rnorm = nullptr;   // L2 norm of every resident row (cosine metric), roundup(max_n, 64) floats
    uint16_t *corpus16 = nullptr;  // bf16 copy, max_n x max_d (after rt_enable_filtered)
    uint32_t *bad16 = nullptr;     // set by the conversion when a value is not finite in bf16
    float *err16 = nullptr;        // per row, an upper bound on |row - bf16 copy| (after rt_enable_filtered)
    uint8_t *corpus8 = nullptr;    // e4m3 codes of each row / its scale, max_n x max_d (after rt_enable_filtered)
    float2 *meta8 = nullptr;       // per row {power-of-two scale s, the row's part of the fp8 bound}
    uint32_t *bad8 = nullptr;      // set by the conversion when a value is not finite
    bool copy8_ok = false;         // the fp8 copy matches the resident corpus and is usable
    bool copy16_ok = false;        // the bf16 copy matches the resident corpus and is usable
};

struct rt_engine {
    int device = 0;
    int num_cus = 0;
    rt_resident *res = nullptr;
    int32_t max_k = 0, max_q = 0;
    float *scores = nullptr;  // batched scores, max_q x roundup(max_n, 64); only when max_q > 1
    float *tmax = nullptr;    // per-query maxima of 32-row score tiles, max_q x tile_ld; only when max_q > 1
    int64_t tile_ld = 0;
    uint64_t *tree = nullptr;       // kTreeRanks merge-tree ranks
    uint32_t *counters = nullptr;   // kMaxQ x kMaxWgsPerSeg arrival counters
    float *ubuf = nullptr;          // filtered search: max_q x roundup(max_n, 64) upper bounds
    float *thr = nullptr;           // filtered search: max_q thresholds
    uint64_t *cand = nullptr;       // batched filtered search, large k: max_q x roundup(max_n, 64) candidate ranks
    uint32_t *cand_cnt = nullptr;   // max_q x kMaxCollectWaves: ranks per wave's slice of cand
    int32_t filter_storage = RT_FILTER_AUTO;  // first pass of a single-query filtered search
    int32_t filter_path = RT_FILTER_PATH_NONE;  // what the last filtered call ran
    hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
    bool profiling = false;
    bool had_batch_kernel = false;
    bool dirty = false;
    int32_t last_hip = 0;
};

namespace rt {
bool engine_filtered_ready(const rt_engine *e) { return e != nullptr && e->ubuf != nullptr; }
}  // namespace rt

static rt_status hip_fail(rt_engine *e, hipError_t err) {
    if (e) {
        e->last_hip = (int32_t)err;
        e->dirty = true;
    }
    (void)hipGetLastError();
    return RT_EHIP;
}

extern "C" {

rt_status rt_filter_bounds(int32_t d, float *out2) {
    if (d < 1 || out2 == nullptr) return RT_EINVAL;
    out2[0] = rt::filter_bound_factor(d);
    out2[1] = rt::filter_underflow_slack(d);
    return RT_OK;
}

rt_status rt_filter_cosine_bounds(int32_t known, float a, float e, float qnorm, float rnorm, float *out2) {
    if (out2 == nullptr) return RT_EINVAL;
    float hi = INFINITY, lo = -INFINITY;
    rt::cosine_bounds(known != 0, a, e, qnorm, rnorm, hi, lo);
    out2[0] = hi;
    out2[1] = lo;
    return RT_OK;
}

float rt_cosine_score(float acc, float qnorm, float rnorm) { return rt::cosine_of(acc, qnorm, rnorm); }

rt_status rt_filter_bounds_fp8(int32_t d, float *out3) {
    if (d < 1 || out3 == nullptr) return RT_EINVAL;
    rt::filter_bound_constants_fp8(d, &out3[0], &out3[1], &out3[2]);
    return RT_OK;
}

rt_status rt_set_filter_storage(rt_engine *e, int32_t storage) {
    if (!e || (storage != RT_FILTER_AUTO && storage != RT_FILTER_BF16 && storage != RT_FILTER_FP8)) return RT_EINVAL;
    e->filter_storage = storage;
    return RT_OK;
}

int32_t rt_filter_path_used(const rt_engine *e) { return e ? e->filter_path : RT_FILTER_PATH_NONE; }

rt_status rt_filter_bounds_batched(int32_t d, float *out3) {
    if (d < 1 || out3 == nullptr) return RT_EINVAL;
    rt::filter_bound_constants_batched(d, &out3[0], &out3[1], &out3[2]);
    return RT_OK;
}

void rt_engine_destroy(rt_engine *e) {
    if (!e) return;
    int prev = 0;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(e->device);
    (void)hipDeviceSynchronize();
    (void)hipFree(e->scores);
    (void)hipFree(e->tmax);
    (void)hipFree(e->tree);
    (void)hipFree(e->counters);
    (void)hipFree(e->ubuf);
    (void)hipFree(e->thr);
    (void)hipFree(e->cand);
    (void)hipFree(e->cand_cnt);
    for (auto &ev : e->ev)
        if (ev) (void)hipEventDestroy(ev);
    if (e->res && e->res->refs.fetch_sub(1) == 1) {
        (void)hipFree(e->res->corpus);
        (void)hipFree(e->res->rnorm);
        (void)hipFree(e->res->corpus16);
        (void)hipFree(e->res->bad16);
        (void)hipFree(e->res->err16);
        (void)hipFree(e->res->corpus8);
        (void)hipFree(e->res->meta8);
        (void)hipFree(e->res->bad8);
        delete e->res;
    }
    (void)hipSetDevice(prev);
    delete e;
}

static bool dev_alloc(void **p, size_t bytes) {
    if (hipMalloc(p, bytes) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return true;
}

// Allocate and initialise an engine's own scratch (everything but the resident
// corpus) on the current device; e->res, device, max_k and max_q are set.
static rt_status setup_scratch(rt_engine *e) {
    hipError_t err = hipDeviceGetAttribute(&e->num_cus, hipDeviceAttributeMultiprocessorCount, e->device);
    if (err != hipSuccess || e->num_cus < 1) e->num_cus = 256;
    (void)hipGetLastError();
    const int64_t max_n = e->res->max_n;
    const int64_t ld = (max_n + 63) / 64 * 64;
    e->tile_ld = ((max_n + 31) / 32 + 63) / 64 * 64;
    bool ok = dev_alloc(reinterpret_cast<void **>(&e->tree), sizeof(uint64_t) * (size_t)kTreeRanks) &&
              dev_alloc(reinterpret_cast<void **>(&e->counters), sizeof(uint32_t) * (size_t)(kMaxQ * kMaxWgsPerSeg));
    if (ok && e->max_q > 1)
        ok = dev_alloc(reinterpret_cast<void **>(&e->scores), sizeof(float) * (size_t)e->max_q * (size_t)ld) &&
             dev_alloc(reinterpret_cast<void **>(&e->tmax), sizeof(float) * (size_t)e->max_q * (size_t)e->tile_ld);
    if (!ok) return RT_ENOMEM;
    err = hipMemset(e->counters, 0, sizeof(uint32_t) * (size_t)(kMaxQ * kMaxWgsPerSeg));
    if (err == hipSuccess) err = rt::prepare_mfma_scores();
    if (err == hipSuccess) err = rt::prepare_mfma_filter();
    for (int i = 0; i < 4 && err == hipSuccess; ++i) err = hipEventCreate(&e->ev[i]);
    if (err == hipSuccess) err = hipDeviceSynchronize();
    if (err != hipSuccess) {
        (void)hipGetLastError();
        return RT_EHIP;
    }
    return RT_OK;
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
    rt_resident *r = new (std::nothrow) rt_resident();
    if (!e || !r) {
        delete e;
        delete r;
        return RT_ENOMEM;
    }
    e->device = device;
    e->max_k = max_k;
    e->max_q = max_q;
    e->res = r;
    r->max_n = max_n;
    r->max_d = max_d;
    int prev = 0;
    (void)hipGetDevice(&prev);
    hipError_t err = hipSetDevice(device);
    if (err != hipSuccess) {
        rt_engine_destroy(e);
        return hip_fail(nullptr, err);
    }
    const int64_t ld = (max_n + 63) / 64 * 64;
    st = (dev_alloc(reinterpret_cast<void **>(&r->corpus), sizeof(float) * (size_t)max_n * (size_t)max_d) &&
          dev_alloc(reinterpret_cast<void **>(&r->rnorm), sizeof(float) * (size_t)ld))
             ? RT_OK
             : RT_ENOMEM;
    if (st == RT_OK && hipMemset(r->rnorm, 0, sizeof(float) * (size_t)ld) != hipSuccess) st = RT_EHIP;
    if (st == RT_OK) st = setup_scratch(e);
    (void)hipSetDevice(prev);
    if (st != RT_OK) {
        rt_engine_destroy(e);
        (void)hipGetLastError();
        return st;
    }
    *out = e;
    return RT_OK;
}

rt_status rt_engine_create_shared(rt_engine *other, int32_t max_k, int32_t max_q, rt_engine **out) {
    if (out == nullptr) return RT_EINVAL;
    *out = nullptr;
    if (other == nullptr) return RT_EINVAL;
    rt_status st = rt_check_create(other->res->max_n, other->res->max_d, max_k, max_q);
    if (st != RT_OK) return st;
    rt_engine *e = new (std::nothrow) rt_engine();
    if (!e) return RT_ENOMEM;
    e->device = other->device;
    e->max_k = max_k;
    e->max_q = max_q;
    e->res = other->res;
    e->res->refs.fetch_add(1);
    int prev = 0;
    (void)hipGetDevice(&prev);
    hipError_t err = hipSetDevice(e->device);
    st = (err == hipSuccess) ? setup_scratch(e) : RT_EHIP;
    (void)hipSetDevice(prev);
    if (st != RT_OK) {
        rt_engine_destroy(e);
        (void)hipGetLastError();
        return st;
    }
    *out = e;
    return RT_OK;
}

// Rebuild the bf16 copy of the resident rows (synchronous); *ok tells whether
// every value is finite in bf16, so that the filtered search's bounds hold.
static hipError_t refresh_copy16(rt_resident *r, int64_t n, int32_t d, int num_cus, bool *ok) {
    *ok = false;
    hipError_t err = hipMemset(r->bad16, 0, sizeof(uint32_t));
    if (err == hipSuccess) err = rt::launch_to_bf16(r->corpus, r->corpus16, n * (int64_t)d, r->bad16, num_cus, nullptr);
    if (err == hipSuccess) err = rt::launch_bf16_row_errors(r->corpus, n, d, r->err16, num_cus, nullptr);
    uint32_t bad = 1;
    if (err == hipSuccess) err = hipMemcpy(&bad, r->bad16, sizeof(uint32_t), hipMemcpyDeviceToHost);
    if (err == hipSuccess) *ok = (bad == 0);
    return err;
}

// Rebuild the fp8 copy (synchronous); *ok tells whether it is usable (a depth
// with an fp8 first pass and every value finite).
static hipError_t refresh_copy8(rt_resident *r, int64_t n, int32_t d, int num_cus, bool *ok) {
    *ok = false;
    if (!rt::fp8_search_ok(d)) return hipSuccess;
    hipError_t err = hipMemset(r->bad8, 0, sizeof(uint32_t));
    if (err == hipSuccess)
        err = rt::launch_to_fp8(r->corpus, n, d, r->rnorm, r->corpus8, r->meta8, r->bad8, num_cus, nullptr);
    uint32_t bad = 1;
    if (err == hipSuccess) err = hipMemcpy(&bad, r->bad8, sizeof(uint32_t), hipMemcpyDeviceToHost);
    if (err == hipSuccess) *ok = (bad == 0);
    return err;
}

rt_status upload_corpus_rowmajor(rt_engine *e, const float *corpus, int64_t n, int32_t d) {
    if (!e) return RT_EINVAL;
    rt_resident *r = e->res;
    rt_status st = rt_check_upload(r->max_n, r->max_d, corpus, n, d);
    if (st != RT_OK) return st;
    int prev = 0;
    (void)hipGetDevice(&prev);
    hipError_t err = hipSetDevice(e->device);
    if (err == hipSuccess)
        err = hipMemcpy(r->corpus, corpus, sizeof(float) * (size_t)n * (size_t)d, hipMemcpyDefault);
    // The rows' L2 norms for the cosine metric and the filtered search,
    // computed once per upload.
    if (err == hipSuccess) err = rt::launch_row_norms(r->corpus, n, d, r->rnorm, e->num_cus, nullptr);
    r->copy16_ok = false;
    r->copy8_ok = false;
    bool ok16 = false, ok8 = false;
    if (err == hipSuccess && r->corpus16) err = refresh_copy16(r, n, d, e->num_cus, &ok16);
    if (err == hipSuccess && r->corpus8) err = refresh_copy8(r, n, d, e->num_cus, &ok8);
    if (err == hipSuccess) err = hipDeviceSynchronize();
    (void)hipSetDevice(prev);
    if (err != hipSuccess) {
        r->n = 0;
        r->d = 0;
        return hip_fail(e, err);
    }
    r->n = n;
    r->d = d;
    r->copy16_ok = ok16;
    r->copy8_ok = ok8;
    return RT_OK;
}

rt_status rt_enable_filtered(rt_engine *e) {
    if (!e) return RT_EINVAL;
    rt_resident *r = e->res;
    int prev = 0;
    (void)hipGetDevice(&prev);
    hipError_t err = hipSetDevice(e->device);
    rt_status st = RT_OK;
    const int64_t ld = (r->max_n + 63) / 64 * 64;
    if (err == hipSuccess && !r->corpus16) {
        if (!dev_alloc(reinterpret_cast<void **>(&r->corpus16),
                       sizeof(uint16_t) * (size_t)r->max_n * (size_t)r->max_d) ||
            !dev_alloc(reinterpret_cast<void **>(&r->bad16), sizeof(uint32_t)) ||
            !dev_alloc(reinterpret_cast<void **>(&r->err16), sizeof(float) * (size_t)ld)) {
            (void)hipFree(r->corpus16);
            (void)hipFree(r->bad16);
            (void)hipFree(r->err16);
            r->corpus16 = nullptr;
            r->bad16 = nullptr;
            r->err16 = nullptr;
            st = RT_ENOMEM;
        } else if (r->n > 0) {
            bool ok16 = false;
            err = refresh_copy16(r, r->n, r->d, e->num_cus, &ok16);
            if (err == hipSuccess) r->copy16_ok = ok16;
        }
    }
    if (err == hipSuccess && st == RT_OK && !r->corpus8) {
        if (!dev_alloc(reinterpret_cast<void **>(&r->corpus8), (size_t)r->max_n * (size_t)r->max_d) ||
            !dev_alloc(reinterpret_cast<void **>(&r->meta8), sizeof(float2) * (size_t)ld) ||
            !dev_alloc(reinterpret_cast<void **>(&r->bad8), sizeof(uint32_t))) {
            (void)hipFree(r->corpus8);
            (void)hipFree(r->meta8);
            (void)hipFree(r->bad8);
            r->corpus8 = nullptr;
            r->meta8 = nullptr;
            r->bad8 = nullptr;
            st = RT_ENOMEM;
        } else if (r->n > 0) {
            bool ok8 = false;
            err = refresh_copy8(r, r->n, r->d, e->num_cus, &ok8);
            if (err == hipSuccess) r->copy8_ok = ok8;
        }
    }
    if (err == hipSuccess && st == RT_OK && !e->ubuf) {
        if (!dev_alloc(reinterpret_cast<void **>(&e->ubuf), sizeof(float) * (size_t)e->max_q * (size_t)ld) ||
            !dev_alloc(reinterpret_cast<void **>(&e->thr), sizeof(float) * (size_t)e->max_q)) {
            (void)hipFree(e->ubuf);
            (void)hipFree(e->thr);
            e->ubuf = nullptr;
            e->thr = nullptr;
            st = RT_ENOMEM;
        }
    }
    // Batches with large k re-rank into per-query candidate lists long enough
    // for every row (set-up: the counts start at zero).
    if (err == hipSuccess && st == RT_OK && e->max_q > 1 && !e->cand) {
        if (!dev_alloc(reinterpret_cast<void **>(&e->cand), sizeof(uint64_t) * (size_t)e->max_q * (size_t)ld) ||
            !dev_alloc(reinterpret_cast<void **>(&e->cand_cnt),
                       sizeof(uint32_t) * (size_t)e->max_q * (size_t)kMaxCollectWaves)) {
            (void)hipFree(e->cand);
            (void)hipFree(e->cand_cnt);
            e->cand = nullptr;
            e->cand_cnt = nullptr;
            st = RT_ENOMEM;
        }
    }
    (void)hipSetDevice(prev);
    if (err != hipSuccess) return hip_fail(e, err);
    return st;
}

static rt::TreeLaunch tree_for(rt_engine *e, const Plan &p, int kp, int k, int mode, int32_t *out_idx,
                               void *out_val, const void *src, int64_t src_stride) {
    return rt::tree_launch(e->tree, e->counters, p.wgs, p, kp, k, mode, out_idx, out_val, src, src_stride);
}

static hipError_t prologue(rt_engine *e, hipStream_t s) {
    hipError_t err = hipSuccess;
    if (e->dirty) {
        err = rt::launch_zero_counters(e->counters, (int64_t)kMaxQ * kMaxWgsPerSeg, s);
        if (err != hipSuccess) return err;
        e->dirty = false;
    }
    if (e->profiling) err = hipEventRecord(e->ev[0], s);
    return err;
}

rt_status search_resident_metric(rt_engine *e, const float *queries, int32_t q, int32_t k, int32_t metric,
                                 int32_t *out_idx, float *out_scores, void *stream) {
    if (!e) return RT_EINVAL;
    rt_status st =
        rt_check_search_metric(e->max_k, e->max_q, e->res->n, queries, q, k, metric, out_idx, out_scores);
    if (st != RT_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int prev = 0;
    (void)hipGetDevice(&prev);
    hipError_t err = hipSetDevice(e->device);
    const int64_t n = e->res->n;
    const int d = e->res->d;
    const float *corpus = e->res->corpus;
    const int kp = kp_for(k);
    const float *rnorm = (metric == RT_METRIC_COSINE) ? e->res->rnorm : nullptr;
    const bool batched = q > 1 && e->scores != nullptr && d % 4 == 0 && d <= rt::kMfmaMaxD;
    e->had_batch_kernel = batched;
    if (err == hipSuccess) err = prologue(e, s);
    if (err == hipSuccess && batched) {
        const int64_t ld = (n + 63) / 64 * 64;
        err = rt::launch_mfma_scores(corpus, n, d, queries, q, rnorm, e->scores, ld, e->tmax, e->tile_ld,
                                     e->num_cus, s);
        if (err == hipSuccess && e->profiling) err = hipEventRecord(e->ev[3], s);
        if (err == hipSuccess)
            err = rt::launch_tile_bound_select(e->scores, ld, n, e->tmax, e->tile_ld, q, k, out_idx, out_scores, s);
    } else if (err == hipSuccess) {
        const Plan p = plan_stream(n, q, kp, min_rows_per_wave(d), e->num_cus, kScoreWavesPerCu, rt::gemv_waves(kp));
        const rt::TreeLaunch t = tree_for(e, p, kp, k, 1, out_idx, out_scores, nullptr, 0);
        err = rt::launch_gemv_topk(corpus, n, d, queries, rnorm, q, p.per_wave, p.wgs, t, s);
    }
    if (err == hipSuccess && e->profiling) err = hipEventRecord(e->ev[1], s);
    (void)hipSetDevice(prev);
    if (err != hipSuccess) return hip_fail(e, err);
    return RT_OK;
}

rt_status search_resident(rt_engine *e, const float *queries, int32_t q, int32_t k, int32_t *out_idx,
                          float *out_scores, void *stream) {
    return search_resident_metric(e, queries, q, k, RT_METRIC_DOT, out_idx, out_scores, stream);
}

rt_status search_resident_filtered_metric(rt_engine *e, const float *queries, int32_t q, int32_t k, int32_t metric,
                                          int32_t *out_idx, float *out_scores, void *stream) {
    if (!e) return RT_EINVAL;
    rt_status st =
        rt_check_search_metric(e->max_k, e->max_q, e->res->n, queries, q, k, metric, out_idx, out_scores);
    if (st != RT_OK) return st;
    if (!e->ubuf) return RT_ESTATE;  // rt_enable_filtered was not called on this engine
    rt_resident *r = e->res;
    const int64_t n = r->n;
    const int d = r->d;
    const bool cosine = metric == RT_METRIC_COSINE;
    const bool small_auto = q == 1 && e->filter_storage == RT_FILTER_AUTO && n * (int64_t)d < kFilteredMinElements;
    if (!r->copy16_ok || !rt::filtered_search_ok(d) || small_auto) {
        // the same answers through the plain scan, one query at a time (a plain
        // batch sums in another order)
        e->filter_path = RT_FILTER_PATH_PLAIN;
        for (int32_t i = 0; i < q && st == RT_OK; ++i)
            st = search_resident_metric(e, queries + (int64_t)i * d, 1, k, metric, out_idx + (int64_t)i * k,
                                        out_scores + (int64_t)i * k, stream);
        return st;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    int prev = 0;
    (void)hipGetDevice(&prev);
    hipError_t err = hipSetDevice(e->device);
    const int kp = kp_for(k);
    const int64_t uld = (r->max_n + 63) / 64 * 64;
    // A batch on an engine with batch buffers: bounds for all queries from one
    // bf16 MFMA pass over the copy, per-query thresholds from tile maxima
    // (inner product; a cosine batch takes the single-query passes, one
    // segment per query).
    const bool batched = !cosine && q > 1 && e->tmax != nullptr && rt::mfma_filter_ok(d);
    e->had_batch_kernel = false;
    if (err == hipSuccess) err = prologue(e, s);
    if (err == hipSuccess && batched) {
        e->filter_path = RT_FILTER_PATH_BF16_MATRIX;
        err = rt::launch_mfma_bound(r->corpus16, n, d, queries, q, r->rnorm, r->err16, e->ubuf, e->tmax,
                                    e->tile_ld, e->num_cus, s);
        if (err == hipSuccess && e->profiling) err = hipEventRecord(e->ev[3], s);
        if (err == hipSuccess) err = rt::launch_tile_threshold(e->tmax, e->tile_ld, n, q, k, e->thr, s);
        // k > 256: per-wave candidate slices and one sort per query beat lists
        // of 512 or 1024 entries per wave and their merge tree (500k x 768, 32
        // queries, threshold + re-rank: 55 against 65 us at k = 257, 74 against
        // 97 us at k = 1024); at k <= 256 the selectors are faster (52 against
        // 54 us at k = 256).
        const bool collect = e->cand != nullptr && kp >= 512;
        if (err == hipSuccess && collect) {
            const Plan pc = plan_stream(n, q, 64, 512, e->num_cus, kBatchRerankWavesPerCu, rt::gemv_waves(64));
            const rt::TreeLaunch tc = tree_for(e, pc, 64, 1, 1, nullptr, nullptr, nullptr, 0);  // selectors idle
            rt::FilterLaunch f;
            f.cb = 0.f;
            f.delta = 0.f;
            f.ubuf = e->ubuf;
            f.uld = uld;
            f.thr = e->thr;
            f.ub16 = reinterpret_cast<const uint16_t *>(e->ubuf);  // tile-major, q queries per tile
            f.ub_tq = q;
            f.cand = e->cand;
            f.cand_ld = uld;
            f.cand_cnt = e->cand_cnt;
            f.cnt_ld = kMaxCollectWaves;
            err = rt::launch_filtered_collect(r->corpus, n, d, queries, q, pc.per_wave, pc.wgs, tc, f, s);
            if (err == hipSuccess)
                err = rt::launch_candidate_select(e->cand, uld, e->cand_cnt, kMaxCollectWaves,
                                                  pc.wgs * rt::collect_waves(), pc.per_wave, q, k, out_idx,
                                                  out_scores, s);
        } else if (err == hipSuccess) {
            const Plan p2 = plan_stream(n, q, kp, 512, e->num_cus, kBatchRerankWavesPerCu, rt::gemv_waves(kp));
            const rt::TreeLaunch t2 = tree_for(e, p2, kp, k, 1, out_idx, out_scores, nullptr, 0);
            rt::FilterLaunch f;  // pass 2 reads only the bounds and thresholds
            f.cb = 0.f;
            f.delta = 0.f;
            f.ubuf = e->ubuf;
            f.uld = uld;
            f.thr = e->thr;
            f.ub16 = reinterpret_cast<const uint16_t *>(e->ubuf);  // tile-major, q queries per tile
            f.ub_tq = q;
            err = rt::launch_filtered_pass2(r->corpus, n, d, queries, q, p2.per_wave, p2.wgs, t2, f, s);
        }
        e->had_batch_kernel = e->profiling;
    } else if (err == hipSuccess) {
        // The fp8 first pass reads a quarter of the fp32 bytes but lets far more
        // rows through to the re-rank (a wider bound): chosen for large corpora,
        // or when the engine asks for it.
        const bool fp8 = r->copy8_ok && rt::fp8_search_ok(d) &&
                         (e->filter_storage == RT_FILTER_FP8 ||
                          (e->filter_storage == RT_FILTER_AUTO && n * (int64_t)d >= kFp8MinElements));
        const Plan p1 = plan_stream(n, q, kp, 32, e->num_cus, kScoreWavesPerCu, rt::gemv_waves(kp));
        const Plan p2 = plan_stream(n, q, kp, 512, e->num_cus, kScoreWavesPerCu, rt::gemv_waves(kp));
        const rt::TreeLaunch t1 = tree_for(e, p1, kp, k, 3, nullptr, e->thr, nullptr, 0);
        const rt::TreeLaunch t2 = tree_for(e, p2, kp, k, 1, out_idx, out_scores, nullptr, 0);
        rt::FilterLaunch f;
        f.cb = rt::filter_bound_factor(d);
        f.delta = rt::filter_underflow_slack(d);
        f.ubuf = e->ubuf;
        f.uld = uld;
        f.thr = e->thr;
        f.crn = cosine ? r->rnorm : nullptr;
        // 16-bit upper bounds (rounded up): half the pass's writes, which cost
        // more than reads next to a full-rate read stream (1M x 1024: fp8 pass
        // 174.0 -> 169.8 us, bf16 pass 322.9 -> 317.3 us)
        f.bounds16 = true;
        e->had_batch_kernel = e->profiling;
        if (fp8) {
            e->filter_path = RT_FILTER_PATH_FP8;
            err = rt::launch_filtered_search8(r->corpus, r->corpus8, r->meta8, n, d, queries, q,
                                              p1.per_wave, p1.wgs, t1, p2.per_wave, p2.wgs, t2, f,
                                              e->profiling ? e->ev[3] : nullptr, s);
        } else {
            e->filter_path = RT_FILTER_PATH_BF16;
            err = rt::launch_filtered_search(r->corpus, r->corpus16, r->rnorm, n, d, queries, q, p1.per_wave, p1.wgs,
                                             t1, p2.per_wave, p2.wgs, t2, f, e->profiling ? e->ev[3] : nullptr, s);
        }
    }
    if (err == hipSuccess && e->profiling) err = hipEventRecord(e->ev[1], s);
    (void)hipSetDevice(prev);
    if (err != hipSuccess) return hip_fail(e, err);
    return RT_OK;
}

rt_status search_resident_filtered(rt_engine *e, const float *queries, int32_t q, int32_t k, int32_t *out_idx,
                                   float *out_scores, void *stream) {
    return search_resident_filtered_metric(e, queries, q, k, RT_METRIC_DOT, out_idx, out_scores, stream);
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
    const Plan p = rt::plan_select(values, n, kp, e->num_cus, kTreeRanks, kMaxWgsPerSeg);
    const rt::TreeLaunch t = tree_for(e, p, kp, k, 2, out_idx, out_values, values, 0);
    if (err == hipSuccess) err = rt::launch_select_topk(values, 0, n, dtype, 1, p.per_wave, p.wgs, t, s);
    if (err == hipSuccess && e->profiling) err = hipEventRecord(e->ev[1], s);
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
    if (err == hipSuccess && e->had_batch_kernel) err = hipEventElapsedTime(&ms3[1], e->ev[0], e->ev[3]);
    if (err != hipSuccess) {
        e->last_hip = (int32_t)err;
        (void)hipGetLastError();
        return RT_EHIP;
    }
    ms3[2] = ms3[0] - ms3[1];
    return RT_OK;
}

rt_status rt_read_probe(rt_engine *e, int32_t reps, void *stream, float *out_ms) {
    if (!e || !out_ms || reps < 1) return RT_EINVAL;
    rt_resident *r = e->res;
    if (r->n < 1) return RT_ESTATE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int prev = 0;
    (void)hipGetDevice(&prev);
    hipError_t err = hipSetDevice(e->device);
    const int64_t n16 = r->n * (int64_t)r->d / 4;
    // the merge-tree array (kTreeRanks words, rewritten by every search) takes any per-wave word
    uint32_t *sink = reinterpret_cast<uint32_t *>(e->tree);
    if (err == hipSuccess) err = hipEventRecord(e->ev[0], s);
    for (int32_t i = 0; i < reps && err == hipSuccess; ++i)
        err = rt::launch_read_probe(r->corpus, n16, sink, e->num_cus, s);
    if (err == hipSuccess) err = hipEventRecord(e->ev[1], s);
    if (err == hipSuccess) err = hipEventSynchronize(e->ev[1]);
    float ms = 0.f;
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, e->ev[0], e->ev[1]);
    e->had_batch_kernel = false;
    (void)hipSetDevice(prev);
    if (err != hipSuccess) return hip_fail(e, err);
    *out_ms = ms / (float)reps;
    return RT_OK;
}

rt_status rt_engine_info(const rt_engine *e, int64_t *out7) {
    if (!e || !out7) return RT_EINVAL;
    out7[0] = e->res->max_n;
    out7[1] = e->res->max_d;
    out7[2] = e->max_k;
    out7[3] = e->max_q;
    out7[4] = e->res->n;
    out7[5] = e->res->d;
    out7[6] = e->device;
    return RT_OK;
}

}  // extern "C"
