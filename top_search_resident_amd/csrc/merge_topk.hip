// merge_topk.hip -- the merge stage of exact top-K on gfx950.
//
// "GPU-Resident Top-K for Agentic RAG" (A. Banerjee), section 4, Step 4: the
// per-block best-first lists are merged into the global best-K; the top-K of the
// union of per-block top-K lists is the global top-K because anything that beats
// an element inside its block also beats it globally.  The pages walk P cursors
// with one thread; here each workgroup loads up to 8192 ranks (fan_in lists of
// Kp) into LDS and reduces them with a tree of pairwise list merges, each done
// by one wavefront in registers (elementwise max against the reversed partner
// list, then a bitonic merge).  Levels repeat until one list per segment is
// left; the last level writes the K indices and K values (section 4, Step 6
// returns only those 2K numbers) and clears the segment's shared threshold for
// the next call.
#include "kernels.hpp"
#include "wave_topk.hpp"

namespace rt {

template <int R>
__global__ __launch_bounds__(kMergeThreads) void merge_lists_kernel(
    const uint64_t *__restrict__ in_lists, int lists_per_seg, int fan_in, uint64_t *__restrict__ out_lists,
    int mode, int k, int32_t *__restrict__ out_idx, uint32_t *__restrict__ out_val,
    const uint32_t *__restrict__ src, int64_t src_seg_stride, uint64_t *__restrict__ seg_thr) {
    constexpr int Kp = 64 * R;
    extern __shared__ uint64_t sm[];
    const int seg = blockIdx.y;
    const int group = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wv = tid >> 6;
    const int nwaves = blockDim.x >> 6;
    const int first = group * fan_in;
    const int count = (lists_per_seg - first < fan_in) ? lists_per_seg - first : fan_in;

    const uint64_t *src_lists = in_lists + ((int64_t)seg * lists_per_seg + first) * Kp;
    const int live = count * Kp;
    for (int i = tid; i < fan_in * Kp; i += blockDim.x) sm[i] = (i < live) ? src_lists[i] : 0ull;
    __syncthreads();

    for (int s = 1; s < fan_in; s <<= 1) {
        const int pairs = fan_in / (2 * s);
        for (int p = wv; p < pairs; p += nwaves) {
            const int a = p * 2 * s, b = a + s;
            if (b >= count) continue;  // partner is empty: list a is already the result
            uint64_t A[R], B[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                A[r] = sm[a * Kp + r * 64 + lane];
                B[r] = sm[b * Kp + r * 64 + lane];
            }
            list_absorb_list<R>(A, B);
#pragma unroll
            for (int r = 0; r < R; ++r) sm[a * Kp + r * 64 + lane] = A[r];
        }
        __syncthreads();
    }

    if (mode == 0) {
        uint64_t *dst = out_lists + ((int64_t)seg * gridDim.x + group) * Kp;
        for (int i = tid; i < Kp; i += blockDim.x) dst[i] = sm[i];
        return;
    }
    for (int r = tid; r < k; r += blockDim.x) {
        const uint64_t v = sm[r];
        const uint32_t idx = rank_index(v);
        out_idx[(int64_t)seg * k + r] = (int32_t)idx;
        if (mode == 1) {
            out_val[(int64_t)seg * k + r] = __float_as_uint(f32_of_order_key(rank_key(v)));
        } else {
            out_val[(int64_t)seg * k + r] = src[(int64_t)seg * src_seg_stride + idx];
        }
    }
    if (tid == 0) seg_thr[seg] = 0ull;
}

__global__ void reset_thr_kernel(uint64_t *seg_thr, int count) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) seg_thr[i] = 0ull;
}

hipError_t launch_merge(const uint64_t *in_lists, int lists_per_seg, int fan_in, int segments, int kp,
                        uint64_t *out_lists, int mode, int k, int32_t *out_idx, void *out_val, const void *src,
                        int64_t src_seg_stride, uint64_t *seg_thr, hipStream_t stream) {
    const int groups = (lists_per_seg + fan_in - 1) / fan_in;
    const dim3 grid(groups, segments);
    const size_t lds = (size_t)fan_in * kp * sizeof(uint64_t);
    uint32_t *ov = static_cast<uint32_t *>(out_val);
    const uint32_t *sv = static_cast<const uint32_t *>(src);
    switch (kp / 64) {
#define RT_CASE(RR)                                                                                          \
    case RR:                                                                                                 \
        hipLaunchKernelGGL((merge_lists_kernel<RR>), grid, dim3(kMergeThreads), lds, stream, in_lists,        \
                           lists_per_seg, fan_in, out_lists, mode, k, out_idx, ov, sv, src_seg_stride, seg_thr); \
        break;
        RT_CASE(1) RT_CASE(2) RT_CASE(4) RT_CASE(8) RT_CASE(16)
#undef RT_CASE
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_reset(uint64_t *seg_thr, int count, hipStream_t stream) {
    hipLaunchKernelGGL(reset_thr_kernel, dim3((count + 255) / 256), dim3(256), 0, stream, seg_thr, count);
    return hipGetLastError();
}

}  // namespace rt
