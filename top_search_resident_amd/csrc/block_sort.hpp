// block_sort.hpp -- bitonic sort of up to a few thousand 64-bit ranks by one
// workgroup (gfx950), best (largest) first.  Used where a workgroup has
// gathered candidates in LDS: the batched selector's kept scores and the merge
// tree's nodes.
#pragma once
#include "wave_topk.hpp"

namespace rt {

// Sort sm[0 .. M) best-first with the NT threads of the workgroup (M a power of
// two, 64 <= M).  Bitonic network on registers: the first min(M, NT) threads
// hold E = M / NT (at least one) elements, element r * NT + t in thread t.
// Exchanges with a partner in the same wave go through DPP / permlane, partners
// in the same thread are register swaps, and only partners in another wave go
// through LDS -- instead of one LDS round trip and barrier per step.  Every
// thread of the workgroup must call it.
template <int NT, int M>
__device__ __forceinline__ void block_sort_desc_m(uint64_t *sm) {
    constexpr int ACT = M < NT ? M : NT;  // active threads (whole waves)
    constexpr int E = M / ACT;
    const int t = threadIdx.x;
    const bool active = t < ACT;
    uint64_t x[E];
#pragma unroll
    for (int r = 0; r < E; ++r) x[r] = active ? sm[r * ACT + t] : 0ull;
    __syncthreads();
#pragma unroll
    for (int k2 = 2; k2 <= M; k2 <<= 1) {
#pragma unroll
        for (int j = k2 >> 1; j > 0; j >>= 1) {
            if (j >= ACT) {  // partner in this thread: register r ^ (j / ACT)
                const int jr = j / ACT;
#pragma unroll
                for (int r = 0; r < E; ++r) {
                    if ((r & jr) == 0) {
                        const int p = r | jr;
                        const bool desc = (((r * ACT) + t) & k2) == 0;
                        const uint64_t hi = umax64(x[r], x[p]), lo = umin64(x[r], x[p]);
                        x[r] = desc ? hi : lo;
                        x[p] = desc ? lo : hi;
                    }
                }
            } else if (j >= 64) {  // partner in another wave: through LDS
                if (active) {
#pragma unroll
                    for (int r = 0; r < E; ++r) sm[r * ACT + t] = x[r];
                }
                __syncthreads();
                if (active) {
#pragma unroll
                    for (int r = 0; r < E; ++r) {
                        const uint64_t y = sm[r * ACT + (t ^ j)];
                        const bool desc = (((r * ACT) + t) & k2) == 0;
                        const bool lower = (t & j) == 0;
                        x[r] = cmpx64(x[r], y, lower == desc);
                    }
                }
                __syncthreads();
            } else if (active) {  // partner in this wave
#pragma unroll
                for (int r = 0; r < E; ++r) {
                    const uint64_t y = shfl_xor_u64(x[r], j);
                    const bool desc = (((r * ACT) + t) & k2) == 0;
                    const bool lower = (t & j) == 0;
                    x[r] = cmpx64(x[r], y, lower == desc);
                }
            }
        }
    }
    if (active) {
#pragma unroll
        for (int r = 0; r < E; ++r) sm[r * ACT + t] = x[r];
    }
    __syncthreads();
}

// Sort sm[0 .. m) best-first, m a power of two in [64, CAP] (CAP <= 8192).
template <int NT, int CAP>
__device__ __forceinline__ void block_sort_desc_any(uint64_t *sm, int m) {
    switch (m) {
        case 64: block_sort_desc_m<NT, 64>(sm); break;
        case 128: block_sort_desc_m<NT, 128>(sm); break;
        case 256: block_sort_desc_m<NT, 256>(sm); break;
        case 512: block_sort_desc_m<NT, 512>(sm); break;
        case 1024: if constexpr (CAP >= 1024) block_sort_desc_m<NT, 1024>(sm); break;
        case 2048: if constexpr (CAP >= 2048) block_sort_desc_m<NT, 2048>(sm); break;
        case 4096: if constexpr (CAP >= 4096) block_sort_desc_m<NT, 4096>(sm); break;
        default: if constexpr (CAP >= 8192) block_sort_desc_m<NT, 8192>(sm); break;
    }
}

}  // namespace rt
