// select_static.hip -- topk_select_noalloc: the raw-array top-K of topk_select
// for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The kernels are topk_select's (two-stage selection: per-workgroup best-K
// lists, then the merge tree); their scratch -- the merge tree's list storage
// and arrival counters -- lives in one file-scope device array instead of an
// engine's allocations.  Each GPU the library runs on holds its own copy of the
// array until the process ends; its device address is looked up once per
// device (hipGetSymbolAddress with that device current) and only that address
// is ever handed to a kernel.  Every call on a GPU shares the array: calls that
// overlap on one GPU (different streams, or threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/resident_topk.h"
#include "kernels.hpp"
#include "limits.hpp"
#include "plan.hpp"

namespace {

// Merge-tree list storage: 2^19 ranks (4 MiB).  A launch of w workgroups with
// lists of kp entries needs at most 2 w kp ranks, so lists of 1024 entries run
// at most 256 workgroups (the planner caps them).
constexpr int64_t kStaticTreeRanks = int64_t(1) << 19;
// Arrival counters: at most one per workgroup (all levels of the tree together
// use fewer than the workgroup count).
constexpr int64_t kStaticMaxWgs = 2048;
constexpr int32_t kStaticMaxK = rt::kMaxK;
constexpr int kMaxDevices = 64;

struct DeviceScratch {
    uint64_t *tree = nullptr;      // device address of scratch[0 .. kStaticTreeRanks)
    uint32_t *counters = nullptr;  // device address of the counters after it
    int num_cus = 0;
    bool dirty = true;             // counters must be cleared before the next launch
};

DeviceScratch g_dev[kMaxDevices];
std::mutex g_mu;

}  // namespace

// tree ranks, then kStaticMaxWgs 32-bit counters (zero between calls)
static __device__ __align__(256) uint64_t scratch[kStaticTreeRanks + kStaticMaxWgs / 2];

extern "C" rt_status topk_select_noalloc(const void *values, int32_t dtype, int64_t n, int32_t k, int32_t *out_idx,
                                         void *out_values, void *stream) {
    rt_status st = rt_check_select(kStaticMaxK, values, dtype, n, k, out_idx, out_values);
    if (st != RT_OK) return st;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return RT_EHIP;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceScratch &ds = g_dev[dev];
    hipError_t err = hipSuccess;
    if (ds.tree == nullptr) {
        // once per device, with that device current: the array's address on it
        void *ptr = nullptr;
        err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (err != hipSuccess || ptr == nullptr) {
            (void)hipGetLastError();
            return RT_EHIP;
        }
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
        (void)hipGetLastError();
        ds.tree = static_cast<uint64_t *>(ptr);
        ds.counters = reinterpret_cast<uint32_t *>(ds.tree + kStaticTreeRanks);
        ds.num_cus = cus;
        ds.dirty = true;
    }
    if (ds.dirty) {  // first use on this device, or after a failed launch: a fill kernel, no memset
        err = rt::launch_zero_counters(ds.counters, kStaticMaxWgs, s);
        if (err != hipSuccess) {
            (void)hipGetLastError();
            return RT_EHIP;
        }
        ds.dirty = false;
    }
    const int kp = rt::kp_for(k);
    const rt::Plan p = rt::plan_select(values, n, kp, ds.num_cus, kStaticTreeRanks, kStaticMaxWgs);
    const rt::TreeLaunch t =
        rt::tree_launch(ds.tree, ds.counters, p.wgs, p, kp, k, 2, out_idx, out_values, values, 0);
    err = rt::launch_select_topk(values, 0, n, dtype, 1, p.per_wave, p.wgs, t, s);
    if (err != hipSuccess) {
        ds.dirty = true;
        (void)hipGetLastError();
        return RT_EHIP;
    }
    return RT_OK;
}
