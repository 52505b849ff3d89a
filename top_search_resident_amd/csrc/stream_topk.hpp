// stream_topk.hpp -- exact top-K on gfx950 in one kernel launch per call.
//
// "GPU-Resident Top-K for Agentic RAG" (A. Banerjee), section 4: Step 2 scores
// every corpus row by inner product, Step 3 lets each block of rows build its
// own best-K list, Step 4 merges the per-block lists into the global best-K, and
// only K indices and K scores leave (Step 6).  The pages launch three kernels:
// one thread per row for scoring (uncoalesced along D), one thread per block
// for a bubble-sort selection, and one thread for the merge.  Here a single
// kernel does all of it:
//
//   1. streaming: each wavefront reads a contiguous row range with 16-byte
//      non-temporal coalesced loads, reduces each row's dot product across a
//      group of lanes, and feeds the scores into a register-resident best-K
//      list (wave_topk.hpp) -- the N scores never reach HBM;
//   2. the four waves of a workgroup merge their lists into one (LDS);
//   3. merge tree (raw arrays: grouped by arrival order, see
//      arrival_tree_finish): workgroups are grouped `fan` at a time; each workgroup stores
//      its list, and the LAST workgroup of a group to finish (a global atomic
//      counter per group) loads the group's lists, merges them and moves one
//      level up; the last one at the root writes the K outputs.  Nothing waits
//      on anything (a workgroup that is not last simply exits), and each counter
//      is cleared by the workgroup that completes it, ready for the next call.
//      The lists cross XCDs (each XCD has its own L2), so they are written and
//      read with device-coherent (agent-scope) atomic stores and loads, and a
//      workgroup waits for its stores to complete before it arrives at the
//      counter.  A device-scope release fence would do the same job but writes
//      back the whole L2 of the XCD; issued by every workgroup it cost ~0.2 us
//      each, serialised (~95 us per call at 512 workgroups on MI355X).
//
// Exactness of the two stages: the top-K of the union of per-block top-K lists
// is the global top-K (anything that beats an element inside its block beats it
// globally), so the grouping is free.
//
// The raw-array kernel is the two-stage top-K of "CUDA Programming Model Series
// 9: Efficient TopK" (section 2: each block reduces its share to a local top-K;
// section 3: a second stage merges the local results), with vector loads, the
// same register lists and the same merge tree.
#pragma once
#include "kernels.hpp"
#include "wave_topk.hpp"

namespace rt {

struct TreeArgs {
    uint64_t *tree;          // per segment: seg_tree_stride ranks of list storage
    uint32_t *counters;      // per segment: seg_ctr_stride arrival counters (zero between calls)
    int64_t seg_tree_stride;
    int seg_ctr_stride;
    int fan;                 // lists merged per tree node (power of two, fan * kc <= kTreeEntries)
    int kc;                  // list stride in the tree: smallest power of two >= k if k <= 32, else Kp
    int k;
    int mode;                // 1: index + fp32 score from the rank; 2: index + source element;
                             // 3: only the k-th entry's fp32 value, to out_val[seg]
    int32_t *out_idx;        // [segments][k]
    uint32_t *out_val;       // [segments][k]
    const uint32_t *src;     // mode 2: the array the ranks index into
    int64_t src_seg_stride;
    int arrival;             // nonzero: arrival-ordered groups and binned merges (see arrival_tree_finish)
};

__device__ __forceinline__ void write_output(const TreeArgs &ta, int seg, int r, uint64_t v) {
    if (ta.mode == 3) {  // only the k-th entry's value, as fp32
        if (r == ta.k - 1) ta.out_val[seg] = __float_as_uint(f32_of_order_key(rank_key(v)));
        return;
    }
    const uint32_t idx = rank_index(v);
    ta.out_idx[(int64_t)seg * ta.k + r] = (int32_t)idx;
    ta.out_val[(int64_t)seg * ta.k + r] =
        (ta.mode == 1) ? __float_as_uint(f32_of_order_key(rank_key(v))) : ta.src[(int64_t)seg * ta.src_seg_stride + idx];
}

// Merge `count` best-first lists of 64*R ranks held contiguously in LDS at sm
// into sm[0 .. 64*R).  Pairs of lists are merged by one wave each, level by
// level.  A merge is bound by instruction issue (running several pairs side by
// side in one wave measured slower), so merge throughput is the number of
// waves of the workgroup.
template <int R>
__device__ __forceinline__ void merge_lds_lists(uint64_t *sm, int count) {
    constexpr int Kp = 64 * R;
    const int lane = lane_id();
    const int wv = wave_in_group();
    const int nwaves = blockDim.x >> 6;
    for (int s = 1; s < count; s <<= 1) {
        for (int a = wv * 2 * s; a + s < count; a += nwaves * 2 * s) {
            uint64_t A[R], B[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                A[r] = sm[a * Kp + r * 64 + lane];
                B[r] = sm[(a + s) * Kp + r * 64 + lane];
            }
            list_absorb_list<R>(A, B);
#pragma unroll
            for (int r = 0; r < R; ++r) sm[a * Kp + r * 64 + lane] = A[r];
        }
        __syncthreads();
    }
}

// Merge `count` best-first lists of KC entries each (KC a power of two <= 64)
// held at sm[c * KC ..] into sm[0 .. KC): the best KC of their union.  Rounds
// of pairwise merges, one barrier per round; a pair is merged by a group of KC
// lanes (lane i takes the larger of A[i] and B[KC - 1 - i], which leaves the
// best KC of A and B as a bitonic sequence, then log2(KC) exchange steps sort
// it), so a wave merges 64 / KC pairs at once.  Only the first k <= KC entries
// of a list ever matter, so short lists are merged as short lists.
// One exchange step of a bitonic merge at lane distance J (i = lane within the
// group): the lower lane keeps the larger rank.
template <int J>
__device__ __forceinline__ uint64_t merge_step(uint64_t x, int i) {
    return cmpx64(x, xor_u64<J>(x), (i & J) == 0);
}

// Sort a bitonic sequence held by groups of KC lanes (one rank per lane) into
// best-first order: steps at distances KC/2, ..., 1, spelled out so that every
// lane exchange is a fixed DPP / permlane move.
template <int KC>
__device__ __forceinline__ uint64_t group_bitonic_merge(uint64_t x, int i) {
    if constexpr (KC >= 64) x = merge_step<32>(x, i);
    if constexpr (KC >= 32) x = merge_step<16>(x, i);
    if constexpr (KC >= 16) x = merge_step<8>(x, i);
    if constexpr (KC >= 8) x = merge_step<4>(x, i);
    if constexpr (KC >= 4) x = merge_step<2>(x, i);
    if constexpr (KC >= 2) x = merge_step<1>(x, i);
    return x;
}

template <int KC>
__device__ __forceinline__ void merge_short_lists_t(uint64_t *sm, int count) {
    constexpr int PER_WAVE = kWave / KC;
    const int lane = lane_id();
    const int i = lane & (KC - 1);
    const int slots = (int)(blockDim.x >> 6) * PER_WAVE;
    const int slot = wave_in_group() * PER_WAVE + lane / KC;
    for (int s = 1; s < count; s <<= 1) {
        const int pairs = (count - s + 2 * s - 1) / (2 * s);  // lists a = 0, 2s, ... with a + s < count
        for (int p0 = 0; p0 < pairs; p0 += slots) {
            if (p0 + wave_in_group() * PER_WAVE >= pairs) break;  // no pair for this wave (uniform)
            const int p = p0 + slot;
            // Groups without a pair read list 0 (any in-range address) and
            // do not write.
            const bool active = p < pairs;
            const int a = active ? p * 2 * s : 0;
            const int b = active ? a + s : 0;
            uint64_t x = umax64(sm[a * KC + i], sm[b * KC + (KC - 1 - i)]);
            x = group_bitonic_merge<KC>(x, i);
            if (active) sm[a * KC + i] = x;
        }
        __syncthreads();
    }
}

__device__ __forceinline__ void merge_short_lists(uint64_t *sm, int count, int kc) {
    switch (kc) {
        case 1: merge_short_lists_t<1>(sm, count); break;
        case 2: merge_short_lists_t<2>(sm, count); break;
        case 4: merge_short_lists_t<4>(sm, count); break;
        case 8: merge_short_lists_t<8>(sm, count); break;
        case 16: merge_short_lists_t<16>(sm, count); break;
        case 32: merge_short_lists_t<32>(sm, count); break;
        default: merge_short_lists_t<64>(sm, count); break;
    }
}

// LDS words the merges use besides the lists.
constexpr int kSelectBins = 256;
struct alignas(16) MergeScratch {
    int hist[kSelectBins];  // binned merge: entries per key bin, best bin first
    uint32_t wave_hi[16];   // per wave: the largest key seen
    uint32_t wave_lo[16];   // per wave: the largest key of a k-th list entry seen
    int count;              // candidates gathered
    int cut;                // last bin kept
    int kept;               // entries in bins 0 .. cut
    int flag;
    int ticket;             // arrival tree: this workgroup's ticket
};

// Largest 32-bit value over the wave, in every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, xor_u32<1>(v));
    v = max(v, xor_u32<2>(v));
    v = max(v, xor_u32<4>(v));
    v = max(v, xor_u32<8>(v));
    v = max(v, xor_u32<16>(v));
    v = max(v, xor_u32<32>(v));
    return v;
}

// Inclusive prefix sum over the wave's lanes: DPP shifts within each row of
// 16 lanes, then the row totals added in.
__device__ __forceinline__ int wave_prefix_sum(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
    const int r0 = __builtin_amdgcn_readlane(x, 15);
    const int r1 = __builtin_amdgcn_readlane(x, 31);
    const int r2 = __builtin_amdgcn_readlane(x, 47);
    const int row = lane_id() >> 4;
    return x + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// Merge `count` best-first lists (list c at sm[c * stride ..], stride a power
// of two <= 64, only the first k <= stride entries of a list matter; count *
// stride <= kTreeEntries) into sm[0 .. k), best first.
//
// The best k-th entry of any list is a certified bound: that list alone holds
// k entries at or above it, so every entry of the answer has a key at or
// above its key `lo`.  The keys in [lo, largest key] are split into 256 equal
// bins, the entries counted per bin, and the bins taken from the top until
// they hold k entries: only entries of those bins can be in the answer.  When
// at most 64 remain they are gathered at the front of sm and one wave sorts
// them; otherwise (keys packed into few bins: heavy ties, very uneven
// spreads) the lists are merged pairwise as they are.  Exact either way.  For
// evenly spread scores the bins kept hold about k entries, so the cost is a
// few LDS passes instead of log2(count) rounds of 64-bit merging networks.
// Every thread of the workgroup must call it.
template <int NT>
__device__ __forceinline__ void merge_binned(uint64_t *sm, MergeScratch *ms, int count, int stride, int k) {
    static_assert(NT / kWave <= 16 && NT >= kSelectBins, "per-wave bound slots and one bin per thread");
    if (count <= 1) return;  // one list is its own best k
    const int th = threadIdx.x;
    const int lane = lane_id();
    const int wv = wave_in_group();
    constexpr int E = kTreeEntries / NT;
    const int total = count * stride;
    uint64_t v[E];
    uint32_t hi = 0, lo = 0;
#pragma unroll
    for (int u = 0; u < E; ++u) {
        const int i = u * NT + th;
        const int pos = i & (stride - 1);
        v[u] = (i < total && pos < k) ? sm[i] : 0ull;
        hi = max(hi, rank_key(v[u]));
        if (i < total && pos == k - 1) lo = max(lo, rank_key(v[u]));
    }
    if (th < kSelectBins) ms->hist[th] = 0;
    if (th == 0) ms->count = 0;
    hi = wave_max_u32(hi);
    lo = wave_max_u32(lo);
    if (lane == 0) {
        ms->wave_hi[wv] = hi;
        ms->wave_lo[wv] = lo;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) {
        hi = max(hi, ms->wave_hi[w]);
        lo = max(lo, ms->wave_lo[w]);
    }
    const uint32_t range = hi - lo;  // hi >= lo: lo is the key of an entry
    const int shift = (range < kSelectBins) ? 0 : 32 - __clz((int)range) - 8;
    int bin[E];  // best bin first; -1: below lo or not an entry
#pragma unroll
    for (int u = 0; u < E; ++u) {
        const int i = u * NT + th;
        const uint32_t key = rank_key(v[u]);
        bin[u] = (i < total && (i & (stride - 1)) < k && key >= lo)
                     ? kSelectBins - 1 - (int)((key - lo) >> shift)
                     : -1;
        if (bin[u] >= 0) atomicAdd(&ms->hist[bin[u]], 1);
    }
    __syncthreads();
    if (th < kWave) {  // the first bin at which the running count reaches k
        const int4 h = *reinterpret_cast<const int4 *>(&ms->hist[4 * lane]);
        const int own = h.x + h.y + h.z + h.w;
        const int incl = wave_prefix_sum(own);
        const uint64_t reach = __ballot(incl >= k);  // nonzero: at least k entries have a key >= lo
        if (lane == (int)__builtin_ctzll(reach)) {
            int c = incl - own, b = 4 * lane;
            const int hv[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (c < k) {
                    c += hv[q];
                    b = 4 * lane + q;
                }
            }
            ms->cut = b;
            ms->kept = c;
        }
    }
    __syncthreads();
    if (ms->kept > kWave) {  // uniform: too many candidates for one wave's sort
        if (stride < kWave)
            merge_short_lists(sm, count, stride);
        else
            merge_lds_lists<1>(sm, count);
        return;
    }
    const int cut = ms->cut;
    uint64_t keep[E];
    int pass = 0;
#pragma unroll
    for (int u = 0; u < E; ++u) {
        keep[u] = __ballot(bin[u] >= 0 && bin[u] <= cut);
        pass += __popcll(keep[u]);
    }
    int base = 0;
    if (lane == 0 && pass) base = atomicAdd(&ms->count, pass);
    base = __shfl(base, 0);
#pragma unroll
    for (int u = 0; u < E; ++u) {  // sm is only read before the barriers above
        if ((keep[u] >> lane) & 1) sm[base + lanes_below(keep[u])] = v[u];
        base += __popcll(keep[u]);
    }
    __syncthreads();
    const int c = ms->kept;  // k <= c <= 64
    if (th < kWave) {
        const uint64_t x = wave_sort64_desc((lane < c) ? sm[lane] : 0ull);
        sm[lane] = x;
    }
    __syncthreads();
}

// Merge `count` best-first lists of `stride` entries (only the first k matter)
// held at sm[c * stride ..] into sm[0 .. k): with `binned`, the binned
// selection from 32 lists up (a node of 128 lists of 32 entries on one
// 16-wave workgroup: 5.1 -> 2.7 us against seven pairwise rounds), pairwise
// merges otherwise.
template <int R, int NT>
__device__ __forceinline__ void merge_lists(uint64_t *sm, MergeScratch *ms, int count, int stride, int k,
                                            bool binned) {
    if constexpr (R == 1) {
        if (count >= 32 && binned)
            merge_binned<NT>(sm, ms, count, stride, k);
        else if (stride < kWave)
            merge_short_lists(sm, count, stride);
        else
            merge_lds_lists<1>(sm, count);
    } else {
        merge_lds_lists<R>(sm, count);
    }
}

// Load `count` lists of kc entries (the first k of each) from tree storage
// at src into sm with device-coherent loads.  All of a thread's loads are
// issued before any is stored to LDS (a loop of load-then-store pays one
// device round trip per entry).  Ends with a barrier.
template <int NT>
__device__ __forceinline__ void load_lists(uint64_t *sm, const uint64_t *src, int count, int kc, int k) {
    constexpr int E = kTreeEntries / NT;
    uint64_t v[E];
#pragma unroll
    for (int u = 0; u < E; ++u) {
        const int i = u * NT + threadIdx.x;
        v[u] = (i < count * kc && (i & (kc - 1)) < k)
                   ? __hip_atomic_load(&src[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                   : 0ull;
    }
#pragma unroll
    for (int u = 0; u < E; ++u) {
        const int i = u * NT + threadIdx.x;
        if (i < count * kc) sm[i] = v[u];
    }
    __syncthreads();
}

// Store the first k entries of sm as a list at dst (device-coherent), wait
// for the stores to complete, and count this workgroup in at *ctr, whose
// group completes with `expected` arrivals.  Returns (to every thread)
// whether this workgroup completed it; the completing workgroup clears the
// counter (and *also_clear, if given) for the next call.
template <int NT>
__device__ __forceinline__ bool store_and_arrive(const uint64_t *sm, uint64_t *dst, int k, uint32_t *ctr,
                                                 int expected, uint32_t *also_clear, MergeScratch *ms) {
    for (int i = threadIdx.x; i < k; i += NT)
        __hip_atomic_store(&dst[i], sm[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);  // this thread's coherent list stores have completed
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t arrived = atomicAdd(ctr, 1u);
        const int last = (int)(arrived + 1 == (uint32_t)expected);
        if (last) {  // all have arrived: clear for the next call
            __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (also_clear) __hip_atomic_store(also_clear, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        ms->flag = last;
    }
    __syncthreads();
    return ms->flag != 0;
}

// Step 3: a merge tree.  Each workgroup stores the first k entries of its list,
// kc entries apart (kc = the smallest power of two >= k for k <= 32, else the
// list length Kp); workgroups are grouped `fan` = kTreeEntries / kc at a time,
// and the last of a group to arrive (a global arrival counter) loads the
// group's lists, merges them and moves one level up; the last one at the root
// writes the outputs.  Lists of up to 32 entries are merged as short lists
// (merge_short_lists: faster than full 64-entry merges from 64 lists up, and
// the short stride makes the fan wider, e.g. one level of up to 512 lists for
// k <= 8), longer ones with the register networks (merge_lds_lists).
template <int R, int NT>
__device__ __forceinline__ void tree_finish(uint64_t *sm, MergeScratch *ms, const TreeArgs &ta, int seg) {
    const int k = ta.k;
    const int kc = ta.kc;
    int count = gridDim.x;
    uint64_t *base = ta.tree + (int64_t)seg * ta.seg_tree_stride;
    uint32_t *ctr = ta.counters + (int64_t)seg * ta.seg_ctr_stride;
    int node = blockIdx.x;
    int64_t level_off = 0;
    int ctr_off = 0;
    while (true) {
        const int parent = node / ta.fan;
        const int first = parent * ta.fan;
        const int children = (count - first < ta.fan) ? count - first : ta.fan;
        if (!store_and_arrive<NT>(sm, base + level_off + (int64_t)node * kc, k, &ctr[ctr_off + parent], children,
                                  nullptr, ms))
            return;
        load_lists<NT>(sm, base + level_off + (int64_t)first * kc, children, kc, k);
        merge_lists<R, NT>(sm, ms, children, kc, k, ta.arrival != 0);
        const int up = (count + ta.fan - 1) / ta.fan;
        if (up == 1) {
            for (int r = threadIdx.x; r < k; r += NT) write_output(ta, seg, r, sm[r]);
            return;
        }
        level_off += (int64_t)count * kc;
        ctr_off += up;
        node = parent;
        count = up;
    }
}

// The merge tree above makes the last workgroup to finish climb every level
// of it, merging a full group at each.  When the grid needs more than one
// level, the groups are formed by arrival order instead, so that the last
// workgroups to finish merge little.  Each workgroup takes a ticket (0 for the
// first to finish) as it finishes streaming.  Counting back from the last
// ticket, r = count - 1 - ticket: r = 0 is a group of one, r in [2^j, 2^(j+1))
// a group of 2^j while 2^j < fan, and the earlier tickets form groups of fan.
// A group's last member to arrive merges the group's lists (a group of one
// skips this); the group results are merged by the last group to complete,
// which writes the outputs.  With ~count / fan + log2(fan) + 1 groups, the
// last workgroup to finish typically stores its list and merges a dozen
// lists, while the big groups were merged as their members arrived.
struct ArrivalGroup {
    int g;        // group number
    int first_r;  // first member, counted back from the last ticket
    int size;     // members
};

__device__ __forceinline__ ArrivalGroup arrival_group(int r, int count, int fan) {
    ArrivalGroup a;
    if (r == 0) {
        a.g = 0;
        a.first_r = 0;
        a.size = 1;
    } else if (r < fan) {
        const int j = 31 - __clz(r);
        a.g = j + 1;
        a.first_r = 1 << j;
        a.size = 1 << j;
    } else {
        const int q = (r - fan) / fan;
        a.g = (31 - __clz(fan)) + 1 + q;
        a.first_r = fan + q * fan;
        a.size = fan;
    }
    if (a.first_r + a.size > count) a.size = count - a.first_r;
    return a;
}

// Groups for `count` workgroups; the arrival tree is used when the position
// tree would need two levels or more and the group results fit one merge:
// counters [0, groups) per group, [groups] for the group results, [groups + 1]
// for the tickets.
__device__ __forceinline__ int arrival_groups(int count, int fan) { return arrival_group(count - 1, count, fan).g + 1; }
__device__ __forceinline__ bool use_arrival_tree(const TreeArgs &ta, int count) {
    if (!ta.arrival || count <= ta.fan) return false;
    const int groups = arrival_groups(count, ta.fan);
    return groups <= ta.fan && groups + 2 <= ta.seg_ctr_stride;
}

template <int R, int NT>
__device__ __forceinline__ void arrival_tree_finish(uint64_t *sm, MergeScratch *ms, const TreeArgs &ta, int seg,
                                                    int ticket) {
    const int k = ta.k;
    const int kc = ta.kc;
    const int count = gridDim.x;
    const int groups = arrival_groups(count, ta.fan);
    uint64_t *base = ta.tree + (int64_t)seg * ta.seg_tree_stride;  // [count] ticket lists, then [groups] results
    uint32_t *ctr = ta.counters + (int64_t)seg * ta.seg_ctr_stride;
    uint64_t *const results = base + (int64_t)count * kc;
    const ArrivalGroup a = arrival_group(count - 1 - ticket, count, ta.fan);
    if (a.size > 1) {
        if (!store_and_arrive<NT>(sm, base + (int64_t)ticket * kc, k, &ctr[a.g], a.size, nullptr, ms)) return;
        const int first_ticket = count - a.first_r - a.size;
        load_lists<NT>(sm, base + (int64_t)first_ticket * kc, a.size, kc, k);
        merge_lists<R, NT>(sm, ms, a.size, kc, k, true);
    }
    if (!store_and_arrive<NT>(sm, results + (int64_t)a.g * kc, k, &ctr[groups], groups, &ctr[groups + 1], ms))
        return;
    load_lists<NT>(sm, results, groups, kc, k);
    merge_lists<R, NT>(sm, ms, groups, kc, k, true);
    for (int r = threadIdx.x; r < k; r += NT) write_output(ta, seg, r, sm[r]);
}

// Steps 2 and 3 above.  `sm` is kTreeEntries ranks of LDS; NT the workgroup size.
template <int R, int NT>
__device__ __forceinline__ void finish_workgroup(WaveSelector<R> &sel, uint64_t *sm, MergeScratch *ms,
                                                 const TreeArgs &ta, int seg) {
    constexpr int Kp = 64 * R;
    const int lane = lane_id();
    const int wv = wave_in_group();
    const bool arrival = use_arrival_tree(ta, gridDim.x);

    // 2. the workgroup's wave lists -> one list in sm[0 .. Kp) (NT / 64 * Kp <= kTreeEntries).
#pragma unroll
    for (int r = 0; r < R; ++r) sm[wv * Kp + r * 64 + lane] = sel.L[r];
    __syncthreads();
    // Every wave has finished streaming: take the arrival ticket.  Its round
    // trip overlaps the workgroup's merge (an increment: the compiler waits
    // for an add's result at once, to spread it over the wave's lanes).
    uint32_t ticket = 0;
    if (arrival && threadIdx.x == 0)
        ticket = atomicInc(&ta.counters[(int64_t)seg * ta.seg_ctr_stride + arrival_groups(gridDim.x, ta.fan) + 1],
                           0xffffffffu);
    merge_lists<R, NT>(sm, ms, NT / 64, Kp, ta.k, ta.arrival != 0);
    if (gridDim.x == 1) {
        for (int r = threadIdx.x; r < ta.k; r += NT) write_output(ta, seg, r, sm[r]);
        return;
    }
    // 3. across the workgroups of this segment.
    if (arrival) {
        if (threadIdx.x == 0) ms->ticket = (int)ticket;
        __syncthreads();
        arrival_tree_finish<R, NT>(sm, ms, ta, seg, ms->ticket);
    } else {
        tree_finish<R, NT>(sm, ms, ta, seg);
    }
}

// ---------------------------------------------------------------- scoring

// Per-lane part of an fp32 row's inner product: the FMA chain over this lane's
// L float4 columns (components x, y, z, w, in order), columns past the row end
// masked to zero (their bits are and-ed with a zero mask: a select or branch on
// a loaded register makes the compiler wait for every outstanding load first).
// group_sum of it over the row's lane group is the row's score.  Every kernel
// that scores fp32 rows with a lane-group shape goes through this function, so
// they all compute the same bits for the same row.
template <int G, int L>
__device__ __forceinline__ float lane_chain(const float4 (&x)[L], const float4 (&qv)[L],
                                            const uint32_t (&cmask)[L]) {
    float a = 0.f;
#pragma unroll
    for (int j = 0; j < L; ++j) {
        float4 v = x[j];
        if constexpr (G * L > 4) {  // a shape that can be padded
            v.x = __uint_as_float(__float_as_uint(v.x) & cmask[j]);
            v.y = __uint_as_float(__float_as_uint(v.y) & cmask[j]);
            v.z = __uint_as_float(__float_as_uint(v.z) & cmask[j]);
            v.w = __uint_as_float(__float_as_uint(v.w) & cmask[j]);
        }
        a = fmaf(v.x, qv[j].x, a);
        a = fmaf(v.y, qv[j].y, a);
        a = fmaf(v.z, qv[j].z, a);
        a = fmaf(v.w, qv[j].w, a);
    }
    return a;
}

// Rows each lane group takes per step: one, or two for rows of a single float4
// per lane.
template <int L>
struct RowUnroll {
    static constexpr int value = (L == 1) ? 2 : 1;
};

// A group of G = 2^LG lanes owns one row at a time; lane g of the group loads
// float4 columns g, g+G, ..., g+(L-1)G of that row, so a row is covered by one
// instruction per j and consecutive lanes read consecutive 16 B.  Columns past
// the row end (when G*L > d/4) are loaded from the last column and replaced by
// 0, so every load is unconditional.  Every row is reduced in exactly the same
// order (per-lane FMA chain over j and the four components, then group_sum), so
// identical rows get bit-identical scores wherever they sit, and exact ties
// resolve by index.
// Loads: with P = 0 a step issues its loads and consumes them at once, so a
// wave has one step in flight -- best when each wave streams hundreds of rows
// and the chip is bandwidth-bound (measured on MI355X at 1M x 1024: any
// lookahead costs 1-2%).  With P > 0 loads run P steps ahead: slot s of a ring
// of P register sets holds step i + s; it is consumed in place and refilled
// with step i + s + P, so every wait is a counted wait for one slot's loads --
// best when each wave has only tens of rows and every step would otherwise pay
// a full memory latency (50k x 768: 42 -> 34 us).  Rows past the wave's range
// are loaded from its last row (cached) and never offered, so no load is
// predicated.
// COS selects the cosine metric: each wave computes the query's norm once, the
// rows' norms (rnorm, computed at upload) are loaded with the rows, and each
// dot product becomes cosine_of(dot, |q|, |row|) before it is ranked.
template <int LG, int L, int R, bool COS, int P>
__global__ __launch_bounds__(64 * gemv_waves(64 * R)) void gemv_topk_kernel(
    const float *__restrict__ corpus, int64_t n, int d, const float *__restrict__ queries,
    const float *__restrict__ rnorm, int64_t rows_per_wave, TreeArgs ta) {
    constexpr int G = 1 << LG;
    constexpr int RPS = 64 >> LG;  // rows per lane-group pass
    constexpr int U = RowUnroll<L>::value;
    constexpr int STEP = RPS * U;  // rows per wave step
    constexpr int SLOTS = P > 0 ? P : 1;
    constexpr int W = gemv_waves(64 * R);
    __shared__ uint64_t stage[W][128];
    __shared__ uint64_t sm[kTreeEntries];
    __shared__ MergeScratch ms;

    const int seg = blockIdx.y;
    const int lane = lane_id();
    const int wv = wave_in_group();
    const int64_t wave = (int64_t)blockIdx.x * W + wv;
    const int g = lane & (G - 1);
    const int h = lane >> LG;
    const int d4 = d >> 2;
    const float4 *__restrict__ q4 = reinterpret_cast<const float4 *>(queries + (int64_t)seg * d);
    uint64_t *const my_stage = stage[wv];

    WaveSelector<R> sel;
    sel.init(ta.k);

    float qnorm = 0.f;
    if constexpr (COS) qnorm = wave_l2_norm(queries + (int64_t)seg * d, d);

    // Columns past the row end (G * L > d / 4) load the last column; their bits
    // are and-ed with a zero mask (a plain select or branch on a loaded register
    // makes the compiler wait for every outstanding load first).
    float4 qv[L];
    int colc[L];
    uint32_t cmask[L];
#pragma unroll
    for (int j = 0; j < L; ++j) {
        const int col = j * G + g;
        colc[j] = (col < d4) ? col : d4 - 1;
        cmask[j] = (col < d4) ? 0xffffffffu : 0u;
        qv[j] = (col < d4) ? q4[col] : make_float4(0.f, 0.f, 0.f, 0.f);
    }

    const int64_t r_begin = wave * rows_per_wave;
    const int64_t r_end = (r_begin + rows_per_wave < n) ? r_begin + rows_per_wave : n;
    if (r_begin < r_end) {
        const float4 *__restrict__ c4 = reinterpret_cast<const float4 *>(corpus);
        const int64_t last = r_end - 1;
        float4 x[SLOTS][U][L];
        float rn[SLOTS][U];
        // Fill slot s with the rows of the step starting at row r0.
        auto load_step = [&](int s, int64_t r0) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                int64_t row = r0 + u * RPS + h;
                row = row < last ? row : last;
                const float4 *p = c4 + row * d4;
#pragma unroll
                for (int j = 0; j < L; ++j) x[s][u][j] = load_nt(p + colc[j]);
                if constexpr (COS) rn[s][u] = rnorm[row];
            }
        };
        // Score the rows of slot s (step starting at row rs) and offer them;
        // with P > 0 the slot is refilled with step rs + P * STEP first.
        auto consume = [&](int s, int64_t rs) {
            float acc[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                acc[u] = group_sum(lane_chain<G, L>(x[s][u], qv, cmask), LG);
                if constexpr (COS) acc[u] = cosine_of(acc[u], qnorm, rn[s][u]);
            }
            if constexpr (P > 0) {
                load_step(s, rs + P * STEP);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t row = rs + u * RPS + h;
                const bool valid = (g == 0) && (row < r_end);
                const uint64_t rank = make_rank(order_key_f32(acc[u]), (uint32_t)row);
                sel.offer(my_stage, rank, valid && rank > sel.thr);
            }
        };
        if constexpr (P == 0) {
            for (int64_t r0 = r_begin; r0 < r_end; r0 += STEP) {
                load_step(0, r0);
                consume(0, r0);
            }
        } else {
            // The prologue must issue the slots in ring order, as the loop
            // refills them: the wait for slot s at the loop head is computed
            // for the worse of the two orders.
#pragma unroll
            for (int s = 0; s < P; ++s) {
                load_step(s, r_begin + s * STEP);
                __builtin_amdgcn_sched_barrier(0);
            }
            for (int64_t r0 = r_begin; r0 < r_end; r0 += P * STEP) {
#pragma unroll
                for (int s = 0; s < P; ++s) consume(s, r0 + s * STEP);
            }
        }
    }
    sel.finish(my_stage);
    finish_workgroup<R, W * 64>(sel, sm, &ms, ta, seg);
}

// Any d: one row per wave at a time, scalar loads strided by 64 lanes.
template <int R, bool COS>
__global__ __launch_bounds__(64 * gemv_waves(64 * R)) void gemv_topk_generic_kernel(
    const float *__restrict__ corpus, int64_t n, int d, const float *__restrict__ queries,
    const float *__restrict__ rnorm, int64_t rows_per_wave, TreeArgs ta) {
    constexpr int U = 4;
    constexpr int W = gemv_waves(64 * R);
    __shared__ uint64_t stage[W][128];
    __shared__ uint64_t sm[kTreeEntries];
    __shared__ MergeScratch ms;
    const int seg = blockIdx.y;
    const int lane = lane_id();
    const int wv = wave_in_group();
    const int64_t wave = (int64_t)blockIdx.x * W + wv;
    const float *__restrict__ q = queries + (int64_t)seg * d;
    uint64_t *const my_stage = stage[wv];
    float qnorm = 0.f;
    if constexpr (COS) qnorm = wave_l2_norm(q, d);
    WaveSelector<R> sel;
    sel.init(ta.k);
    const int64_t r_begin = wave * rows_per_wave;
    const int64_t r_end = (r_begin + rows_per_wave < n) ? r_begin + rows_per_wave : n;
    for (int64_t r0 = r_begin; r0 < r_end; r0 += U) {
        float acc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) acc[u] = 0.f;
        for (int c = lane; c < d; c += 64) {
            const float qc = q[c];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t row = r0 + u;
                const float x = (row < r_end) ? corpus[row * d + c] : 0.f;
                acc[u] = fmaf(x, qc, acc[u]);
            }
        }
        for (int m = 32; m >= 1; m >>= 1) {
#pragma unroll
            for (int u = 0; u < U; ++u) acc[u] += __shfl_xor(acc[u], m);
        }
        if constexpr (COS) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t row = r0 + u;
                acc[u] = cosine_of(acc[u], qnorm, rnorm[row < r_end ? row : r_end - 1]);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = r0 + u;
            const bool valid = (lane == 0) && (row < r_end);
            const uint64_t rank = make_rank(order_key_f32(acc[u]), (uint32_t)row);
            sel.offer(my_stage, rank, valid && rank > sel.thr);
        }
    }
    sel.finish(my_stage);
    finish_workgroup<R, W * 64>(sel, sm, &ms, ta, seg);
}

// ---------------------------------------------------------------- raw arrays

// Compile-time flag selecting the masked (edge) form of a filtering step.
template <bool B>
struct EdgeTag {
    static constexpr bool value = B;
};

// Segment `seg` is the n-element array at base + seg * seg_stride (32-bit
// elements).  It is read as 16-byte groups of the enclosing aligned range: group
// t holds elements 4t - head .. 4t - head + 3, where head = (address mod 16) / 4.
// Elements outside [0, n) are masked.  An aligned 16-byte group never crosses a
// page, so reading the part of a group outside the array cannot fault.
template <int DT, int R, int W>
__global__ __launch_bounds__(W * 64) void select_topk_kernel(
    const uint32_t *__restrict__ base, int64_t seg_stride, int64_t n, int64_t groups_per_wave, TreeArgs ta) {
    constexpr int U = 2;  // 2 x 16 B per lane per step, loads one step ahead (measured best at 1e8 int32)
    constexpr int kBootM = (R <= 8) ? R : 8;  // keys per lane behind the first step's bound
    __shared__ uint64_t stage[W][128];
    __shared__ uint64_t sm[kTreeEntries];
    __shared__ uint64_t wg_thr;  // largest k-th entry any wave of the workgroup has published
    __shared__ MergeScratch ms;
    const int seg = blockIdx.y;
    const int lane = lane_id();
    const int wv = wave_in_group();
    const int64_t wave = (int64_t)blockIdx.x * W + wv;
    // The array may start anywhere; loads are 16-byte groups from the aligned
    // address at or below its start, `head` elements early.  The pointer is
    // formed from the kernel argument (not from an integer) so that the loads
    // stay global loads, which LDS waits do not have to drain.
    const uint32_t *const seg_base = base + seg * seg_stride;
    const int head = (int)((reinterpret_cast<uintptr_t>(seg_base) & 15u) >> 2);
    const uint4 *__restrict__ a4 = reinterpret_cast<const uint4 *>(seg_base - head);
    const int64_t total_groups = (n + head + 3) >> 2;
    uint64_t *const my_stage = stage[wv];

    WaveSelector<R> sel;
    sel.init(ta.k);
    if (threadIdx.x == 0) wg_thr = 0ull;
    __syncthreads();
    const int64_t g_begin = wave * groups_per_wave;
    const int64_t g_end = (g_begin + groups_per_wave < total_groups) ? g_begin + groups_per_wave : total_groups;

    // One step: U groups of 4 elements per lane.  EDGE steps mask elements
    // outside [0, n) and groups past g_end; interior steps skip those tests.
    auto step = [&](int64_t g0, const uint4 (&v)[U], auto edge_tag) {
        constexpr bool EDGE = decltype(edge_tag)::value;
        uint32_t key[U][4];
        uint32_t mx = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                key[u][c] = (DT == 0) ? order_key_i32((int32_t)e[c]) : order_key_f32(__uint_as_float(e[c]));
                if constexpr (EDGE) {
                    const int64_t grp = g0 + u * 64 + lane;
                    const int64_t idx = grp * 4 + c - head;
                    if (!(grp < g_end && idx >= 0 && idx < n)) key[u][c] = 0;  // below every threshold key but 0
                }
                mx = key[u][c] > mx ? key[u][c] : mx;
            }
        }
        // First step of the wave: start from a certified bound instead of an
        // empty list.  Each lane's M-th largest key km has M elements at or
        // above it; the q-th largest km over the wave (q = ceil(k / M) <= 64)
        // then has q * M >= k elements at or above it, so no element with a
        // smaller key can be in the top k.  Masked slots hold key 0 and only
        // weaken the bound.
        if constexpr (kBootM > 0) {
            if (g0 == g_begin) {
                static_assert(U * 4 == 8, "bootstrap reads eight keys per lane");
                const uint32_t flat[8] = {key[0][0], key[0][1], key[0][2], key[0][3],
                                          key[1][0], key[1][1], key[1][2], key[1][3]};
                const int q = (ta.k + kBootM - 1) / kBootM;
                if (q <= 64) {
                    const uint32_t sorted = wave_sort64_desc_u32(mth_largest8<kBootM>(flat));
                    const uint32_t kk = (uint32_t)__builtin_amdgcn_readlane((int)sorted, q - 1);
                    const uint64_t boot = ((uint64_t)kk << 32) - 1;  // keeps every key >= kk
                    if (kk != 0 && boot > sel.thr) sel.thr = boot;
                }
            }
        }
        sel.sync_shared(&wg_thr);
        const uint32_t thr_key = rank_key(sel.thr);
        // A key below the threshold's key can never enter the list (key ties go
        // to the exact rank test).  Most steps stop here; in the others only the
        // element slots that hold a candidate pay for the exact test.
        if (__ballot(mx >= thr_key) == 0) return;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t grp = g0 + u * 64 + lane;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int64_t idx = grp * 4 + c - head;
                bool maybe = key[u][c] >= rank_key(sel.thr);
                if constexpr (EDGE) maybe = maybe && grp < g_end && idx >= 0 && idx < n;
                if (__ballot(maybe) == 0) continue;
                const uint64_t rank = make_rank(key[u][c], (uint32_t)idx);
                sel.offer(my_stage, rank, maybe && rank > sel.thr, &wg_thr);
            }
        }
    };

    // Loads run one step ahead of the filtering.  Groups past the range reload
    // the last group (masked in edge steps).
    uint4 nv[U];
    if (g_begin < g_end) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t grp = g_begin + u * 64 + lane;
            nv[u] = load_nt(a4 + ((grp < g_end) ? grp : g_end - 1));
        }
    }
    for (int64_t g0 = g_begin; g0 < g_end; g0 += 64 * U) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = nv[u];
        if (g0 + 64 * U < g_end) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t grp = g0 + 64 * U + u * 64 + lane;
                nv[u] = load_nt(a4 + ((grp < g_end) ? grp : g_end - 1));
            }
        }
        // Every element of an interior step is in range: no group past g_end, no
        // element before the array start or past its end.
        const bool interior = (g0 + 64 * U <= g_end) && (g0 > 0 || head == 0) && ((g0 + 64 * U) * 4 - head <= n);
        if (interior)
            step(g0, v, EdgeTag<false>{});
        else
            step(g0, v, EdgeTag<true>{});
    }
    sel.finish(my_stage, &wg_thr);
    finish_workgroup<R, W * 64>(sel, sm, &ms, ta, seg);
}

// ---------------------------------------------------------------- per-list-size launchers

inline TreeArgs make_tree(const TreeLaunch &t, bool arrival = false) {
    TreeArgs ta;
    ta.tree = t.tree;
    ta.counters = t.counters;
    ta.seg_tree_stride = t.seg_tree_stride;
    ta.seg_ctr_stride = t.seg_ctr_stride;
    ta.kc = tree_stride(t.k, t.kp);
    ta.fan = kTreeEntries / ta.kc;
    ta.k = t.k;
    ta.mode = t.mode;
    ta.out_idx = t.out_idx;
    ta.out_val = static_cast<uint32_t *>(t.out_val);
    ta.src = static_cast<const uint32_t *>(t.src);
    ta.src_seg_stride = t.src_seg_stride;
    ta.arrival = arrival;
    return ta;
}

// (LG, L) pairs the planner can pick for d / 4 in [1, 512] (see pick_group).
#define RT_GEMV_SHAPES(X) \
    X(0, 1) X(0, 3) X(1, 1) X(1, 3) X(2, 1) X(2, 3) X(3, 1) X(3, 3) X(4, 1) X(4, 3) X(5, 1) X(5, 3) \
    X(6, 1) X(6, 2) X(6, 3) X(6, 4) X(6, 6) X(6, 8)

// Scoring launcher for lists of 64*R entries: the vector kernel of shape (lg, L)
// when `fast`, else the scalar kernel; COS selects the cosine metric (rnorm then
// holds the corpus rows' L2 norms).
template <int R, bool COS>
hipError_t launch_gemv_r(bool fast, int lg, int L, dim3 grid, hipStream_t s, const float *corpus, int64_t n, int d,
                         const float *queries, const float *rnorm, int64_t per_wave, const TreeLaunch &t) {
    // Lookahead only for short row ranges per wave (see gemv_topk_kernel).
    const bool ahead = per_wave <= kGemvLookaheadRows;
    const TreeArgs ta = make_tree(t);
    const dim3 block(64 * gemv_waves(64 * R));
    if (!fast) {
        hipLaunchKernelGGL((gemv_topk_generic_kernel<R, COS>), grid, block, 0, s, corpus, n, d, queries, rnorm,
                           per_wave, ta);
        return hipGetLastError();
    }
#define RT_SHAPE(LGV, LV)                                                                                      \
    if (lg == LGV && L == LV) {                                                                                \
        if (ahead)                                                                                             \
            hipLaunchKernelGGL((gemv_topk_kernel<LGV, LV, R, COS, 2>), grid, block, 0, s, corpus, n, d, queries, \
                               rnorm, per_wave, ta);                                                           \
        else                                                                                                   \
            hipLaunchKernelGGL((gemv_topk_kernel<LGV, LV, R, COS, 0>), grid, block, 0, s, corpus, n, d, queries, \
                               rnorm, per_wave, ta);                                                           \
        return hipGetLastError();                                                                              \
    }
    RT_GEMV_SHAPES(RT_SHAPE)
#undef RT_SHAPE
    return hipErrorInvalidValue;
}

// Raw-array selection launcher for lists of 64*R entries (dtype 0 = int32, 1 = fp32).
template <int R>
hipError_t launch_select_r(int dtype, dim3 grid, hipStream_t s, const void *data, int64_t n, int64_t seg_stride,
                           int64_t per_wave, const TreeLaunch &t) {
    // Raw arrays: one long stream per wave whose workgroups finish over a
    // spread of several microseconds, which the arrival-ordered tree turns
    // into merges done early (1e8 int32, K = 20 / 50: 77.2 / 80.2 -> 75.1 /
    // 78.4 us).  The scorers' short streams finish together, and there it
    // measured slower (50k x 768, K = 32: 36.8 -> 39.3 us).
    const TreeArgs ta = make_tree(t, true);
    constexpr int W = select_waves(64 * R);
    const uint32_t *base = static_cast<const uint32_t *>(data);
    if (dtype == 0)
        hipLaunchKernelGGL((select_topk_kernel<0, R, W>), grid, dim3(64 * W), 0, s, base, seg_stride, n, per_wave, ta);
    else
        hipLaunchKernelGGL((select_topk_kernel<1, R, W>), grid, dim3(64 * W), 0, s, base, seg_stride, n, per_wave, ta);
    return hipGetLastError();
}

}  // namespace rt
