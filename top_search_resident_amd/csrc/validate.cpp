// validate.cpp -- status names and the host-side argument checks of the C ABI
// (include/resident_topk.h).  Plain C++ with no HIP dependency: the library
// links it, and the CPU test suite also builds it on its own with the address
// and undefined-behaviour sanitizers.  Every entry point runs the matching
// check before it enqueues anything, so an argument error leaves outputs and
// device state untouched.
#include <stdint.h>

#include "../../include/resident_topk.h"
#include "limits.hpp"

using rt::kMaxD;
using rt::kMaxK;
using rt::kMaxN;
using rt::kMaxQ;

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

rt_status rt_check_search_metric(int32_t max_k, int32_t max_q, int64_t resident_n, const void *queries,
                                 int32_t q, int32_t k, int32_t metric, const void *out_idx, const void *out_scores) {
    if (metric != RT_METRIC_DOT && metric != RT_METRIC_COSINE) return RT_EINVAL;
    return rt_check_search(max_k, max_q, resident_n, queries, q, k, out_idx, out_scores);
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

}  // extern "C"
