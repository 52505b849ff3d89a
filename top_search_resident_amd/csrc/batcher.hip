// batcher.hip -- dynamic batching of concurrent single-query searches.
//
// "GPU-Resident Top-K for Agentic RAG" (A. Banerjee), section 1: many small
// agents retrieve against one shared corpus, each with its own query; section
// 9 lists the absence of concurrency between queries inside one engine among
// the engine's limits.  Each single-query scan streams the whole corpus, so
// queries that arrive together are better served by one pass over the corpus
// for all of them.  A batcher collects single-query requests from any number
// of host threads into batches of up to 32 and runs each batch as one batched
// search on its engine:
//
//   exact mode: search_resident_filtered, whose batch path bounds every
//     (row, query) pair with bf16 matrix cores and re-scores the surviving rows
//     with the single-query scan's own arithmetic -- each request gets, bit for
//     bit, the answer the plain single-query scan gives;
//   plain mode: search_resident, whose batch path scores on fp32 matrix cores
//     (scores equal to the single-query scan's within fp32 rounding).
//
// A request's top-k is the first k entries of its batch's top-kmax (kmax the
// largest k in the batch): the comparator is a total order, so the best k are a
// prefix of the best kmax.
//
// One dispatcher thread per batcher waits for the first request, then keeps
// collecting until the batch is full or the first request has waited
// max_wait_us; it stages the batch's queries in pinned memory, runs the search
// on the batcher's own stream, copies the answers back and wakes the waiting
// callers.  Nothing else calls the engine while the batcher exists.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <condition_variable>
#include <cstring>
#include <deque>
#include <memory>
#include <mutex>
#include <new>
#include <thread>
#include <unordered_map>
#include <vector>

#include "limits.hpp"
#include "resident_topk.h"

namespace rt {
// engine.hip: whether rt_enable_filtered has prepared this engine.
bool engine_filtered_ready(const rt_engine *e);
}  // namespace rt

namespace {

using Clock = std::chrono::steady_clock;

struct Request {
    uint64_t ticket = 0;
    std::vector<float> query;  // copied at submission
    int32_t k = 0;
    int32_t *out_idx = nullptr;  // caller's host memory, k entries
    float *out_scores = nullptr;
    Clock::time_point submitted;
    rt_status status = RT_OK;
    bool done = false;
};

}  // namespace

struct rt_batcher {
    rt_engine *e = nullptr;
    int32_t max_batch = 0;
    int32_t max_k = 0;
    int32_t d = 0;
    bool exact = true;
    std::chrono::microseconds max_wait{0};
    int device = 0;
    hipStream_t stream = nullptr;
    float *h_q = nullptr;  // pinned staging: max_batch x d queries
    float *d_q = nullptr;
    int32_t *h_idx = nullptr;  // pinned: max_batch x max_k answers
    float *h_sc = nullptr;
    int32_t *d_idx = nullptr;
    float *d_sc = nullptr;

    std::mutex mu;
    std::condition_variable work;  // a request arrived, or stop
    std::condition_variable done;  // a batch finished
    std::deque<std::shared_ptr<Request>> queue;
    std::unordered_map<uint64_t, std::shared_ptr<Request>> live;  // submitted, not yet waited for
    uint64_t next_ticket = 1;
    bool stop = false;
    int64_t batches = 0, served = 0, largest = 0;
    std::vector<std::shared_ptr<Request>> batch;  // the batch being served (dispatcher only)
    std::thread dispatcher;

    void run();
    void serve(std::vector<std::shared_ptr<Request>> &batch);
};

// One batch: stage the queries, search with k = the batch's largest k, return
// every request's prefix.  Runs on the dispatcher thread without the lock.
void rt_batcher::serve(std::vector<std::shared_ptr<Request>> &batch) {
    const int32_t q = (int32_t)batch.size();
    int32_t kmax = 0;
    for (auto &r : batch) kmax = std::max(kmax, r->k);
    for (int32_t i = 0; i < q; ++i) std::memcpy(h_q + (size_t)i * d, batch[i]->query.data(), sizeof(float) * d);
    rt_status st = RT_OK;
    int64_t info[7];
    if (rt_engine_info(e, info) != RT_OK || info[5] != d || info[4] < kmax) st = RT_ESTATE;  // corpus changed
    hipError_t err = hipSuccess;
    if (st == RT_OK) {
        err = hipMemcpyAsync(d_q, h_q, sizeof(float) * (size_t)q * d, hipMemcpyHostToDevice, stream);
        if (err != hipSuccess) st = RT_EHIP;
    }
    if (st == RT_OK)
        st = exact ? search_resident_filtered(e, d_q, q, kmax, d_idx, d_sc, stream)
                   : search_resident(e, d_q, q, kmax, d_idx, d_sc, stream);
    if (st == RT_OK) {
        err = hipMemcpyAsync(h_idx, d_idx, sizeof(int32_t) * (size_t)q * kmax, hipMemcpyDeviceToHost, stream);
        if (err == hipSuccess)
            err = hipMemcpyAsync(h_sc, d_sc, sizeof(float) * (size_t)q * kmax, hipMemcpyDeviceToHost, stream);
        if (err == hipSuccess) err = hipStreamSynchronize(stream);
        if (err != hipSuccess) st = RT_EHIP;
    }
    if (err != hipSuccess) (void)hipGetLastError();
    for (int32_t i = 0; i < q; ++i) {
        Request &r = *batch[i];
        if (st == RT_OK) {
            std::memcpy(r.out_idx, h_idx + (size_t)i * kmax, sizeof(int32_t) * r.k);
            std::memcpy(r.out_scores, h_sc + (size_t)i * kmax, sizeof(float) * r.k);
        }
        r.status = st;
    }
}

void rt_batcher::run() {
    (void)hipSetDevice(device);
    std::unique_lock<std::mutex> lk(mu);
    while (true) {
        work.wait(lk, [&] { return stop || !queue.empty(); });
        if (queue.empty()) break;  // stop, and everything submitted has been served
        // Collect until the batch is full or its oldest request has waited long enough.
        const Clock::time_point deadline = queue.front()->submitted + max_wait;
        while (!stop && (int32_t)queue.size() < max_batch && Clock::now() < deadline) work.wait_until(lk, deadline);
        batch.clear();  // capacity max_batch, reserved at creation: no allocation here
        while (!queue.empty() && (int32_t)batch.size() < max_batch) {
            batch.push_back(queue.front());
            queue.pop_front();
        }
        lk.unlock();
        serve(batch);
        lk.lock();
        for (auto &r : batch) r->done = true;
        batches += 1;
        served += (int64_t)batch.size();
        largest = std::max<int64_t>(largest, (int64_t)batch.size());
        done.notify_all();
    }
}

extern "C" {

rt_status rt_batcher_create(rt_engine *e, int32_t max_batch, int32_t max_wait_us, int32_t exact, rt_batcher **out) {
    if (out == nullptr) return RT_EINVAL;
    *out = nullptr;
    if (e == nullptr || max_wait_us < 0 || max_wait_us > 1000000 || (exact != 0 && exact != 1)) return RT_EINVAL;
    int64_t info[7];
    rt_status st = rt_engine_info(e, info);  // max_n, max_d, max_k, max_q, resident_n, resident_d, device
    if (st != RT_OK) return st;
    if (max_batch < 1 || max_batch > rt::kMaxQ || max_batch > info[3]) return RT_EINVAL;
    if (info[4] == 0) return RT_ESTATE;  // nothing resident
    std::unique_ptr<rt_batcher> b(new (std::nothrow) rt_batcher());
    if (!b) return RT_ENOMEM;
    b->e = e;
    b->max_batch = max_batch;
    b->max_k = (int32_t)std::min<int64_t>(info[2], info[4]);
    b->d = (int32_t)info[5];
    b->exact = exact != 0;
    b->max_wait = std::chrono::microseconds(max_wait_us);
    b->device = (int)info[6];
    if (b->exact && !rt::engine_filtered_ready(e)) return RT_ESTATE;  // rt_enable_filtered first
    int prev = 0;
    (void)hipGetDevice(&prev);
    hipError_t err = hipSetDevice(b->device);
    const size_t qb = sizeof(float) * (size_t)max_batch * b->d;
    const size_t ab = (size_t)max_batch * b->max_k;
    if (err == hipSuccess) err = hipStreamCreateWithFlags(&b->stream, hipStreamNonBlocking);
    if (err == hipSuccess) err = hipHostMalloc(reinterpret_cast<void **>(&b->h_q), qb, hipHostMallocDefault);
    if (err == hipSuccess) err = hipHostMalloc(reinterpret_cast<void **>(&b->h_idx), sizeof(int32_t) * ab, hipHostMallocDefault);
    if (err == hipSuccess) err = hipHostMalloc(reinterpret_cast<void **>(&b->h_sc), sizeof(float) * ab, hipHostMallocDefault);
    if (err == hipSuccess) err = hipMalloc(reinterpret_cast<void **>(&b->d_q), qb);
    if (err == hipSuccess) err = hipMalloc(reinterpret_cast<void **>(&b->d_idx), sizeof(int32_t) * ab);
    if (err == hipSuccess) err = hipMalloc(reinterpret_cast<void **>(&b->d_sc), sizeof(float) * ab);
    (void)hipSetDevice(prev);
    if (err != hipSuccess) {
        (void)hipGetLastError();
        rt_batcher_destroy(b.release());
        return err == hipErrorOutOfMemory ? RT_ENOMEM : RT_EHIP;
    }
    rt_batcher *raw = b.get();
    try {
        raw->batch.reserve((size_t)max_batch);
        raw->dispatcher = std::thread([raw] { raw->run(); });
    } catch (...) {
        rt_batcher_destroy(b.release());
        return RT_ENOMEM;
    }
    *out = b.release();
    return RT_OK;
}

rt_status rt_batcher_submit(rt_batcher *b, const float *query, int32_t k, int32_t *out_idx, float *out_scores,
                            uint64_t *out_ticket) {
    if (b == nullptr || query == nullptr || out_idx == nullptr || out_scores == nullptr || out_ticket == nullptr)
        return RT_EINVAL;
    if (k < 1 || k > b->max_k) return RT_EINVAL;
    try {  // allocation failures must not cross the C boundary
        auto r = std::make_shared<Request>();
        r->query.assign(query, query + b->d);
        r->k = k;
        r->out_idx = out_idx;
        r->out_scores = out_scores;
        r->submitted = Clock::now();
        {
            std::lock_guard<std::mutex> lk(b->mu);
            if (b->stop) return RT_ESTATE;
            r->ticket = b->next_ticket;
            b->live.emplace(r->ticket, r);
            try {
                b->queue.push_back(r);
            } catch (...) {
                b->live.erase(r->ticket);
                throw;
            }
            b->next_ticket += 1;
            *out_ticket = r->ticket;
        }
        b->work.notify_one();
        return RT_OK;
    } catch (...) {
        return RT_ENOMEM;
    }
}

rt_status rt_batcher_wait(rt_batcher *b, uint64_t ticket) {
    if (b == nullptr) return RT_EINVAL;
    std::unique_lock<std::mutex> lk(b->mu);
    auto it = b->live.find(ticket);
    if (it == b->live.end()) return RT_EINVAL;  // unknown, or already waited for
    std::shared_ptr<Request> r = it->second;
    b->done.wait(lk, [&] { return r->done; });
    b->live.erase(ticket);
    return r->status;
}

rt_status rt_batcher_stats(rt_batcher *b, int64_t *out4) {
    if (b == nullptr || out4 == nullptr) return RT_EINVAL;
    std::lock_guard<std::mutex> lk(b->mu);
    out4[0] = b->batches;
    out4[1] = b->served;
    out4[2] = b->largest;
    out4[3] = (int64_t)b->queue.size();
    return RT_OK;
}

void rt_batcher_destroy(rt_batcher *b) {
    if (b == nullptr) return;
    {
        std::lock_guard<std::mutex> lk(b->mu);
        b->stop = true;
    }
    b->work.notify_all();
    if (b->dispatcher.joinable()) b->dispatcher.join();  // serves what was queued first
    int prev = 0;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(b->device);
    if (b->stream) (void)hipStreamDestroy(b->stream);
    if (b->h_q) (void)hipHostFree(b->h_q);
    if (b->h_idx) (void)hipHostFree(b->h_idx);
    if (b->h_sc) (void)hipHostFree(b->h_sc);
    if (b->d_q) (void)hipFree(b->d_q);
    if (b->d_idx) (void)hipFree(b->d_idx);
    if (b->d_sc) (void)hipFree(b->d_sc);
    (void)hipSetDevice(prev);
    (void)hipGetLastError();
    delete b;
}

}  // extern "C"
