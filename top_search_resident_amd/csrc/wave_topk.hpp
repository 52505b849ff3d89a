// wave_topk.hpp -- wavefront-level (64-lane) exact top-K building blocks for gfx950.
//
// Ordering.  Every candidate is packed into one 64-bit "rank":
//     rank = (order_key(value) << 32) | (0xFFFFFFFF - index)
// order_key is a monotone map of the value to uint32 (larger value -> larger
// key), and the low word is larger for a SMALLER index.  So unsigned 64-bit
// comparison of ranks is exactly the pages' comparator: a larger score wins and
// an exact tie goes to the lower index ("GPU-Resident Top-K for Agentic RAG",
// section 3, "Problem B").  Ranks of distinct elements are distinct, and 0 is
// below every real rank (real low words are >= 0x80000000 because indices are
// < 2^31), so 0 serves as the empty-slot sentinel -- the pages' (-inf, INT_MAX)
// starting point of the merge (section 4, Step 4).
//
// fp32 keys: -0.0 is mapped to +0.0's key, because float equality ties the two.
// int32 keys: flip the sign bit (no negation, so INT32_MIN is safe).
//
// A sorted list of Kp = 64*R ranks lives in registers: entry j is lane (j % 64)
// of register (j / 64), best first.  Candidates are batched 64 at a time,
// bitonic-sorted across the wave and merged into the list with one bitonic merge
// (the pages' per-block selector is an O(K^2) single-lane bubble sort, section 3
// "Problem A"; the 64-lane networks replace it).
#pragma once
#include "cosine_math.hpp"
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rt {

constexpr int kWave = 64;

__device__ __forceinline__ uint32_t order_key_f32(float x) {
    uint32_t b = __float_as_uint(x);
    b = (b == 0x80000000u) ? 0u : b;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float f32_of_order_key(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
__device__ __forceinline__ uint32_t order_key_i32(int32_t x) { return (uint32_t)x ^ 0x80000000u; }

__device__ __forceinline__ uint64_t make_rank(uint32_t key, uint32_t index) {
    return ((uint64_t)key << 32) | (uint64_t)(0xffffffffu - index);
}
__device__ __forceinline__ uint32_t rank_index(uint64_t r) { return 0xffffffffu - (uint32_t)r; }
__device__ __forceinline__ uint32_t rank_key(uint64_t r) { return (uint32_t)(r >> 32); }

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }
// Index of this thread's wave in its workgroup, as a wave-uniform value.
__device__ __forceinline__ int wave_in_group() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Exchange with lane ^ M, without an LDS round trip.  Measured lane semantics on
// gfx950: quad_perm covers M = 1, 2; for M = 4, 8 a lane whose bit M is clear
// reads lane + M (DPP row_shl:M, never crossing its 16-lane row for such a
// lane) and one whose bit is set reads lane - M (row_shr:M);
// v_permlane16_swap / v_permlane32_swap with both operands the same register
// return the two halves of the swap, so lanes pick the half that came from
// lane ^ 16 (^ 32).
template <int M>
__device__ __forceinline__ uint32_t xor_u32(uint32_t v) {
    if constexpr (M == 1) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
    } else if constexpr (M == 2) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
    } else if constexpr (M == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (__lane_id() & 16) ? r[0] : r[1];
    } else if constexpr (M == 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (__lane_id() & 32) ? r[0] : r[1];
    } else {
        static_assert(M == 4 || M == 8, "lane exchange distance");
        const uint32_t up = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x100 + M, 0xF, 0xF, false);
        const uint32_t down = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x110 + M, 0xF, 0xF, false);
        return (__lane_id() & M) ? down : up;
    }
}

template <int M>
__device__ __forceinline__ uint64_t xor_u64(uint64_t v) {
    const uint32_t lo = xor_u32<M>((uint32_t)v);
    const uint32_t hi = xor_u32<M>((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Lane 63 - l: the row mirror (l ^ 15) composed with the 16- and 32-lane swaps.
__device__ __forceinline__ uint64_t reverse_u64(uint64_t v) {
    uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, 0x140, 0xF, 0xF, false);
    uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), 0x140, 0xF, 0xF, false);
    lo = xor_u32<16>(lo);
    hi = xor_u32<16>(hi);
    lo = xor_u32<32>(lo);
    hi = xor_u32<32>(hi);
    return ((uint64_t)hi << 32) | lo;
}

// Runtime-mask form for loops the compiler fully unrolls (the switch folds).
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
    switch (m) {
        case 1: return xor_u64<1>(v);
        case 2: return xor_u64<2>(v);
        case 4: return xor_u64<4>(v);
        case 8: return xor_u64<8>(v);
        case 16: return xor_u64<16>(v);
        case 32: return xor_u64<32>(v);
        default: return v;
    }
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}

// 16-byte streaming loads with the non-temporal hint: the corpus and raw arrays
// are read exactly once per call, so they should not displace reused lines.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_nt(const float4 *p) {
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 load_nt(const uint4 *p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t umin64(uint64_t a, uint64_t b) { return a > b ? b : a; }

// One side of a compare-exchange: the larger of x and its partner y when
// keep_max, else the smaller.  Written as a single compare and a select: the
// form "keep_max ? max(x, y) : min(x, y)" compiles to two compares under
// exec-masked branches, which made every exchange step of the sorting
// networks several times slower.
__device__ __forceinline__ uint64_t cmpx64(uint64_t x, uint64_t y, bool keep_max) {
    const bool x_wins = (x > y) == keep_max;
    return x_wins ? x : y;
}
__device__ __forceinline__ uint32_t cmpx32(uint32_t x, uint32_t y, bool keep_max) {
    const bool x_wins = (x > y) == keep_max;
    return x_wins ? x : y;
}

// Cross-lane moves through DPP (no LDS round trip).  Controls: quad_perm
// [1,0,3,2] and [2,3,0,1] swap neighbours at distance 1 and 2; row_half_mirror
// reverses each 8-lane half-row and row_mirror each 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

__device__ __forceinline__ float readlane_f32(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Sum over each aligned group of G = 2^log2g lanes (log2g <= 6, wave-uniform).
// Steps: neighbours at distance 1 and 2 (quad_perm), then the mirror partner in
// the half-row and in the row -- after the earlier steps every lane of a quad
// (resp. half-row) holds the same value, so the mirror partner stands in for the
// xor partner -- then, for groups wider than a 16-lane row, the row sums are
// read out and added as (r0 + r1) and ((r0 + r1) + (r2 + r3)).  Every group
// is summed in the same fixed order, and every lane of a group ends with the
// group's sum.
__device__ __forceinline__ float group_sum(float v, int log2g) {
    if (log2g >= 1) v += dpp_f32<kDppXor1>(v);
    if (log2g >= 2) v += dpp_f32<kDppXor2>(v);
    if (log2g >= 3) v += dpp_f32<kDppHalfMirror>(v);
    if (log2g >= 4) v += dpp_f32<kDppMirror>(v);
    if (log2g >= 5) {
        const float s01 = readlane_f32(v, 0) + readlane_f32(v, 16);
        const float s23 = readlane_f32(v, 32) + readlane_f32(v, 48);
        if (log2g == 5) {
            v = (lane_id() < 32) ? s01 : s23;
        } else {
            v = s01 + s23;
        }
    }
    return v;
}

// L2 norm of the d floats at v, computed by one whole wave: lane l sums the
// squares of elements l, l + 64, ... in fp64 (each fp32 square is exact in
// fp64), the 64 partial sums are added by a fixed butterfly, and the fp64
// square root is rounded to fp32 once.  Loads are issued eight at a time from
// clamped addresses (out-of-range elements count as zero), so a wave waits for
// one memory latency per 512 elements.  Every wave that calls it on the same
// data gets the same bits, and every lane returns the result.
__device__ __forceinline__ float wave_l2_norm(const float *__restrict__ v, int64_t d) {
    constexpr int B = 8;
    double s = 0.0;
    const int lane = lane_id();
    for (int64_t cb = 0; cb < d; cb += kWave * B) {
        float x[B];
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const int64_t c = cb + i * kWave + lane;
            x[i] = v[c < d ? c : d - 1];
        }
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const double y = (cb + i * kWave + lane < d) ? (double)x[i] : 0.0;
            s = fma(y, y, s);
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
    return (float)sqrt(s);
}

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Make this wave's earlier LDS writes visible to its later LDS reads from other lanes.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Bitonic sort of 64 ranks (one per lane), best first.
__device__ __forceinline__ uint64_t wave_sort64_desc(uint64_t x) {
    const int lane = lane_id();
#pragma unroll
    for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const uint64_t y = shfl_xor_u64(x, j);
            const bool desc_seg = (lane & k) == 0;
            const bool lower = (lane & j) == 0;
            x = cmpx64(x, y, lower == desc_seg);
        }
    }
    return x;
}

// Bitonic sort of 64 keys (one per lane), largest first.
__device__ __forceinline__ uint32_t wave_sort64_desc_u32(uint32_t x) {
    const int lane = lane_id();
#pragma unroll
    for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            uint32_t y;
            switch (j) {
                case 1: y = xor_u32<1>(x); break;
                case 2: y = xor_u32<2>(x); break;
                case 4: y = xor_u32<4>(x); break;
                case 8: y = xor_u32<8>(x); break;
                case 16: y = xor_u32<16>(x); break;
                default: y = xor_u32<32>(x); break;
            }
            const bool desc_seg = (lane & k) == 0;
            const bool lower = (lane & j) == 0;
            x = cmpx32(x, y, lower == desc_seg);
        }
    }
    return x;
}

// The M-th largest (M = 1, 2, 4 or 8) of eight keys.
template <int M>
__device__ __forceinline__ uint32_t mth_largest8(const uint32_t (&in)[8]) {
    uint32_t a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = in[i];
    if constexpr (M == 1) {
        uint32_t m = a[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) m = max(m, a[i]);
        return m;
    } else {
        // bitonic sorting network on 8 registers, largest first
#pragma unroll
        for (int k = 2; k <= 8; k <<= 1) {
#pragma unroll
            for (int j = k >> 1; j > 0; j >>= 1) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int p = i ^ j;
                    if (p > i) {
                        const bool desc = (i & k) == 0;
                        const uint32_t hi = max(a[i], a[p]), lo = min(a[i], a[p]);
                        a[i] = desc ? hi : lo;
                        a[p] = desc ? lo : hi;
                    }
                }
            }
        }
        return a[M - 1];
    }
}

// Sort a bitonic sequence of 64*R ranks (entry j = lane j%64 of register j/64)
// into best-first order.
template <int R>
__device__ __forceinline__ void bitonic_merge_desc(uint64_t (&L)[R]) {
    const int lane = lane_id();
#pragma unroll
    for (int rs = R / 2; rs >= 1; rs >>= 1) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if ((r & rs) == 0) {
                const uint64_t a = L[r], c = L[r + rs];
                L[r] = umax64(a, c);
                L[r + rs] = umin64(a, c);
            }
        }
    }
#pragma unroll
    for (int j = 32; j >= 1; j >>= 1) {
        const bool lower = (lane & j) == 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint64_t y = shfl_xor_u64(L[r], j);
            L[r] = cmpx64(L[r], y, lower);
        }
    }
}

// L := best 64*R of (L u batch); L sorted best-first, batch sorted best-first
// (64 entries, one per lane).  Elementwise max of a descending and an ascending
// sequence keeps the best half and is bitonic.
template <int R>
__device__ __forceinline__ void list_absorb64(uint64_t (&L)[R], uint64_t batch_desc) {
    const uint64_t asc = reverse_u64(batch_desc);  // lane l gets batch[63 - l]
    L[R - 1] = umax64(L[R - 1], asc);
    bitonic_merge_desc<R>(L);
}

// L := best 64*R of (L u M), both sorted best-first with 64*R entries.
template <int R>
__device__ __forceinline__ void list_absorb_list(uint64_t (&L)[R], const uint64_t (&M)[R]) {
#pragma unroll
    for (int r = 0; r < R; ++r) L[r] = umax64(L[r], reverse_u64(M[R - 1 - r]));
    bitonic_merge_desc<R>(L);
}

// Rank of list entry j (0 if the list has fewer than j+1 real entries).  Every
// register is read out with readlane and the wanted one picked among the
// uniform results, so the list is never indexed dynamically (which would push
// it to scratch memory).
template <int R>
__device__ __forceinline__ uint64_t list_entry(const uint64_t (&L)[R], int j) {
    const int reg = j >> 6;
    const int src = j & 63;
    uint64_t v = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint64_t t = readlane_u64(L[r], src);
        v = (r == reg) ? t : v;
    }
    return v;
}

// Per-wave streaming selector.  Candidates are appended to a 128-entry LDS
// staging buffer private to the wave; every 64 of them are sorted and absorbed
// into the register list.  `thr` is a certified bound: some set of k
// already-seen elements all reach or beat it, so anything at or below it can
// never enter the top-k and is not offered.  It is the list's k-th entry (0
// until the list holds k real entries), raised -- when the workgroup shares a
// bound in LDS (`wg_thr`, non-null) -- to the largest k-th entry any wave of
// the workgroup has published.  The staging buffer and the shared bound are
// passed to each call (not stored) so the compiler keeps LDS addressing and
// keeps the list in registers.
// 64-bit word in LDS (address space 3).
typedef __attribute__((address_space(3))) uint64_t lds_u64;

template <int R>
struct WaveSelector {
    uint64_t L[R];
    uint64_t thr;        // wave-uniform
    uint64_t published;  // wave-uniform: last value this wave put into *wg_thr
    int pending;         // wave-uniform
    int k;

    __device__ __forceinline__ void init(int k_) {
#pragma unroll
        for (int r = 0; r < R; ++r) L[r] = 0;
        thr = 0;
        published = 0;
        pending = 0;
        k = k_;
    }

    __device__ __forceinline__ void absorb_stage_front(uint64_t *__restrict__ stage, int count, uint64_t *wg_thr) {
        const int lane = lane_id();
        wave_lds_sync();
        uint64_t x = (lane < count) ? stage[lane] : 0ull;
        x = wave_sort64_desc(x);
        list_absorb64<R>(L, x);
        const uint64_t kth = list_entry<R>(L, k - 1);
        if (kth > thr) thr = kth;
        if (wg_thr != nullptr && kth > published) {
            published = kth;
            if (lane == 0)
                __hip_atomic_fetch_max((lds_u64 *)(wg_thr), kth, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    }

    // Raise thr to the workgroup's shared bound.  The bound lives in LDS; the
    // load is made through an LDS-qualified pointer so that it waits on LDS
    // traffic only, never on the wave's outstanding HBM loads.
    __device__ __forceinline__ void sync_shared(const uint64_t *wg_thr) {
        const uint64_t g = __hip_atomic_load((const lds_u64 *)(wg_thr), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_WORKGROUP);
        if (g > thr) thr = g;
    }

    // Offer one rank per lane; `take` must already include rank > thr.
    __device__ __forceinline__ void offer(uint64_t *__restrict__ stage, uint64_t rank, bool take,
                                          uint64_t *wg_thr = nullptr) {
        const uint64_t m = __ballot(take);
        if (m == 0) return;
        const int lane = lane_id();
        if (take) stage[pending + lanes_below(m)] = rank;
        pending += __popcll(m);
        if (pending >= 64) {
            absorb_stage_front(stage, 64, wg_thr);
            const int rest = pending - 64;
            uint64_t t = 0;
            if (lane < rest) t = stage[64 + lane];
            wave_lds_sync();
            if (lane < rest) stage[lane] = t;
            pending = rest;
        }
    }

    __device__ __forceinline__ void finish(uint64_t *__restrict__ stage, uint64_t *wg_thr = nullptr) {
        if (pending > 0) absorb_stage_front(stage, pending, wg_thr);
        pending = 0;
    }
};

}  // namespace rt
