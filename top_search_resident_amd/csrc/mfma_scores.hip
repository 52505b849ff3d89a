// mfma_scores.hip -- batched inner products on CDNA4 matrix cores.
//
// A batch of q <= 32 queries against the resident corpus is a dense contraction
// S = Q . C^T (q x n, reduction over d).  The pages score one query at a time
// ("GPU-Resident Top-K for Agentic RAG", section 4, Step 2) and list concurrent
// queries as missing (section 9); with a batch the corpus is read from HBM once
// for all queries and the arithmetic runs on v_mfma_f32_32x32x2_f32.
//
// Two kernels.  For the inner product at d in {256, 384, 512, 768} (and n >= 32)
// mfma_scores_dma_kernel below streams the corpus into LDS with direct loads
// and keeps the query block in registers.  Every other batch (cosine, d = 1024,
// other depths) runs the register-staged kernels described here.
//
// Tiling.  One workgroup per CU stages the whole 32 x d query block in LDS,
// zero-padded to a whole number of pipeline rounds of 32 columns (row stride
// padded by 4 floats to spread LDS banks).  Each wave owns tiles of 32 corpus
// rows and produces one 32 x 32 output tile (queries x rows) with
// v_mfma_f32_32x32x2_f32.  For an MFMA step the query operand lane l holds
// Q[l % 32][c] and the corpus operand lane l holds C[row0 + l % 32][c], with the
// column c = c0 + 16 (l / 32) + 4 i + e for step (i, e); so per 32 columns each
// lane issues four 16-byte corpus loads covering 64 contiguous bytes of its row,
// and the two lane halves cover the row's full 128-byte line.  Loads run KPF
// 32-column chunks ahead of the multiplies.  Every load is unconditional:
// addresses past the row end are clamped and their values replaced by zero
// afterwards, rows past n read the last row.  (Predicated loads become
// exec-masked branches, across which the compiler can only wait for all
// outstanding loads, which serialises the pipeline.)  The loads are ordinary
// (cached): a line is consumed by four successive load instructions, and the
// non-temporal hint made it miss again (measured 1.7x slower on MI355X).
// The corpus rows are the MFMA's first (M) operand and the queries its second
// (N), so the 32 x 32 output tile (rows x queries) has element (row, query) in
// lane query % 32 + 32 * ((row / 4) % 2), register (row % 4) + 4 * (row / 8):
// each lane holds sixteen rows of one query, four runs of four consecutive
// rows, stored as four 16-byte stores into that query's score row (row stride
// ld), and the tile's maximum per query is an in-register maximum plus one
// exchange between the lane halves.
#include "kernels.hpp"
#include "lds_dma.hpp"
#include "wave_topk.hpp"

namespace rt {

typedef float floatx16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float comp(const float4 &v, int e) {
    return e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w));
}

// Runtime-depth kernel: chunks of 32 columns loaded ahead of the multiplies and
// independent accumulators (the workgroup size is kMfmaThreads).
constexpr int kMfmaPrefetch = 2;
constexpr int kMfmaAcc = 2;

// Columns the kernel walks for depth d: whole rounds of kpf chunks.
constexpr int mfma_cols(int d, int kpf) { return ((d + 32 * kpf - 1) / (32 * kpf)) * (32 * kpf); }

// Store a finished tile (rows row0 .. row0 + 31 x queries) and, per query, the
// largest of its valid scores into tmax[query][tile].  Lane (query j = lane %
// 32, half h = lane / 32) holds rows 8 g + 4 h + c in register 4 g + c.  With
// COS each inner product is first turned into a cosine with the query's norm
// qn and the rows' norms rn[g] (rows 8 g + 4 h .. + 3).
template <bool COS>
__device__ __forceinline__ void store_tile(const floatx16 &acc_in, int64_t t, int64_t n, int q, int lane,
                                           float *__restrict__ scores, int64_t ld, float *__restrict__ tmax,
                                           int64_t tld, const float4 (&rn)[4], float qn) {
    const int j = lane & 31;
    const int h = lane >> 5;
    const int64_t row0 = t * 32;
    const bool has_q = j < q;
    floatx16 acc = acc_in;
    if constexpr (COS) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            acc[4 * g + 0] = cosine_of(acc[4 * g + 0], qn, rn[g].x);
            acc[4 * g + 1] = cosine_of(acc[4 * g + 1], qn, rn[g].y);
            acc[4 * g + 2] = cosine_of(acc[4 * g + 2], qn, rn[g].z);
            acc[4 * g + 3] = cosine_of(acc[4 * g + 3], qn, rn[g].w);
        }
    }
    float *srow = scores + (int64_t)j * ld + row0 + 4 * h;
    float mx = -INFINITY;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int64_t r = row0 + 8 * g + 4 * h;  // first row of this run of four
        const float4 v = make_float4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
        if (r + 3 < n) {
            if (has_q) *reinterpret_cast<float4 *>(srow + 8 * g) = v;
            mx = fmaxf(mx, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (r + c < n) {
                    if (has_q) srow[8 * g + c] = acc[4 * g + c];
                    mx = fmaxf(mx, acc[4 * g + c]);
                }
            }
        }
    }
    mx = fmaxf(mx, __uint_as_float(xor_u32<32>(__float_as_uint(mx))));
    if (h == 0 && has_q) tmax[(int64_t)j * tld + t] = mx;
}

// Row norms a lane needs for tile t (rows 32 t + 8 g + 4 h .. + 3, g = 0..3).
__device__ __forceinline__ void load_tile_norms(const float *__restrict__ rnorm, int64_t t, int lane,
                                                float4 (&rn)[4]) {
    const float *p = rnorm + t * 32 + 4 * (lane >> 5);
#pragma unroll
    for (int g = 0; g < 4; ++g) rn[g] = *reinterpret_cast<const float4 *>(p + 8 * g);
}

// Per-query L2 norms of the staged query block (row stride dp in LDS), one wave
// per query, into qn[0 .. 32).
__device__ __forceinline__ void stage_query_norms(const float *qs, int dp, int d, float *qn) {
    const int nw = blockDim.x >> 6;
    for (int j = wave_in_group(); j < kMfmaMaxQ; j += nw) {
        const float v = wave_l2_norm(qs + j * dp, d);
        if (lane_id() == 0) qn[j] = v;
    }
}

// KPF: chunks loaded ahead; NT: workgroup size; ACC: independent accumulators
// (chunk j accumulates into acc[j % ACC], summed at the end).
template <int KPF, int NT, int ACC, bool COS>
__global__ __launch_bounds__(NT) void mfma_scores_kernel(const float *__restrict__ corpus, int64_t n, int d,
                                                         const float *__restrict__ queries, int q,
                                                         const float *__restrict__ rnorm,
                                                         float *__restrict__ scores, int64_t ld,
                                                         float *__restrict__ tmax, int64_t tld,
                                                         int64_t tiles_per_wave) {
    static_assert(KPF % ACC == 0, "each ring slot feeds one accumulator");
    extern __shared__ float qs[];
    __shared__ float qn_s[kMfmaMaxQ];
    const int nchunks = (d + 31) / 32;
    const int nck = (nchunks + KPF - 1) / KPF * KPF;  // chunks walked: whole pipeline rounds
    const int dpad = nck * 32;
    const int dp = dpad + 4;
    for (int i = threadIdx.x; i < kMfmaMaxQ * dpad; i += NT) {
        const int r = i / dpad, c = i - r * dpad;
        qs[r * dp + c] = (r < q && c < d) ? queries[(int64_t)r * d + c] : 0.f;
    }
    __syncthreads();
    float qn = 0.f;
    if constexpr (COS) {
        stage_query_norms(qs, dp, d, qn_s);
        __syncthreads();
        qn = qn_s[threadIdx.x & 31];
    }

    const int lane = threadIdx.x & 63;
    const int wv = wave_in_group();  // wave-uniform: the tile loop runs on scalar registers
    const int m = lane & 31;
    const int kk = lane >> 5;
    const int64_t wave = (int64_t)blockIdx.x * (NT / 64) + wv;
    const int64_t tiles = (n + 31) / 32;
    const int64_t t_begin = wave * tiles_per_wave;
    const int64_t t_end = (t_begin + tiles_per_wave < tiles) ? t_begin + tiles_per_wave : tiles;
    const float *qrow = qs + m * dp + 16 * kk;

    for (int64_t t = t_begin; t < t_end; ++t) {
        const int64_t row0 = t * 32;
        const bool valid = row0 + m < n;
        float4 rn[4];
        if constexpr (COS) load_tile_norms(rnorm, t, lane, rn);
        const float *p = corpus + (valid ? row0 + m : n - 1) * (int64_t)d;
        auto load_chunk = [&](int chunk, float4(&dst)[4]) {
            chunk = chunk < nchunks ? chunk : nchunks - 1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int col = chunk * 32 + 16 * kk + 4 * i;
                dst[i] = *reinterpret_cast<const float4 *>(p + (col < d ? col : d - 4));
            }
        };
        floatx16 acc[ACC];
#pragma unroll
        for (int h = 0; h < ACC; ++h)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[h][v] = 0.f;
        float4 buf[KPF][4];
#pragma unroll
        for (int s = 0; s < KPF; ++s) load_chunk(s, buf[s]);
        // Slot s of the ring always holds chunk ci + s: it is consumed in place
        // and then refilled with chunk ci + s + KPF, so no register is copied
        // while a load into it may still be in flight.
        for (int ci = 0; ci < nck; ci += KPF) {
#pragma unroll
            for (int s = 0; s < KPF; ++s) {
                const int c0 = (ci + s) * 32;
                float4 a[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const float4 *>(qrow + c0 + 4 * i);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // Columns past d hold clamped (real) data: select zero there
                    // (a select, not a branch) so the zero query padding
                    // multiplies zeros, whatever the data.
                    const bool in_row = c0 + 16 * kk + 4 * i < d;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[s % ACC] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                            in_row ? comp(buf[s][i], e) : 0.f, comp(a[i], e), acc[s % ACC], 0, 0, 0);
                }
                load_chunk(ci + s + KPF, buf[s]);
                // keep the refill here: left alone, the scheduler sinks it down
                // to its use KPF chunks later, which serialises the loads
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int h = 1; h < ACC; ++h)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[0][v] += acc[h][v];
        store_tile<COS>(acc[0], t, n, q, lane, scores, ld, tmax, tld, rn, qn);
    }
}

// The same tile loop for a depth of exactly d = 32 NCK known at compile time:
// the chunk loop is unrolled, so within a tile every wait for a ring slot is a
// counted wait for that slot's own loads (a loop-carried slot can only be
// waited for with all loads), the column offsets are load immediates with no
// clamping or masking, and the refills of a tile's last chunks already fetch
// the next tile's first chunks (one pipeline across the wave's tiles).
template <int NCK, int KPF, int NT, int ACC, bool COS>
__global__ __launch_bounds__(NT) void mfma_scores_fixed_kernel(const float *__restrict__ corpus, int64_t n,
                                                               const float *__restrict__ queries, int q,
                                                               const float *__restrict__ rnorm,
                                                               float *__restrict__ scores, int64_t ld,
                                                               float *__restrict__ tmax, int64_t tld,
                                                               int64_t tiles_per_wave) {
    static_assert(KPF <= NCK && NCK % ACC == 0, "pipeline shape");
    constexpr int d = NCK * 32;
    constexpr int dp = d + 4;
    extern __shared__ float qs[];
    __shared__ float qn_s[kMfmaMaxQ];
    for (int i = threadIdx.x; i < kMfmaMaxQ * d; i += NT) {
        const int r = i / d, c = i - r * d;
        qs[r * dp + c] = (r < q) ? queries[(int64_t)r * d + c] : 0.f;
    }
    __syncthreads();
    float qn = 0.f;
    if constexpr (COS) {
        stage_query_norms(qs, dp, d, qn_s);
        __syncthreads();
        qn = qn_s[threadIdx.x & 31];
    }

    const int lane = threadIdx.x & 63;
    const int wv = wave_in_group();  // wave-uniform: the tile loop runs on scalar registers
    const int m = lane & 31;
    const int kk = lane >> 5;
    const int64_t wave = (int64_t)blockIdx.x * (NT / 64) + wv;
    const int64_t tiles = (n + 31) / 32;
    const int64_t t_begin = wave * tiles_per_wave;
    const int64_t t_end = (t_begin + tiles_per_wave < tiles) ? t_begin + tiles_per_wave : tiles;
    if (t_begin >= t_end) return;
    const float *qrow = qs + m * dp + 16 * kk;
    auto row_of = [&](int64_t t) {
        const int64_t row = t * 32 + m;
        return corpus + (row < n ? row : n - 1) * (int64_t)d + 16 * kk;
    };
    auto load_chunk = [&](const float *p, int chunk, float4(&dst)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = *reinterpret_cast<const float4 *>(p + chunk * 32 + 4 * i);
    };
    const float *p = row_of(t_begin);
    float4 buf[KPF][4];
#pragma unroll
    for (int s = 0; s < KPF; ++s) load_chunk(p, s, buf[s]);
    // Query operands of the chunk being multiplied; the next chunk's are read
    // from LDS before this chunk's MFMAs are issued, so the MFMAs never wait
    // on an LDS read issued just before them.
    float4 acur[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acur[i] = *reinterpret_cast<const float4 *>(qrow + 4 * i);
    for (int64_t t = t_begin; t < t_end; ++t) {
        const float *pn = (t + 1 < t_end) ? row_of(t + 1) : p;  // past the last tile: reload (cached)
        // The query operands are the same for every tile; an opaque per-tile
        // offset keeps the compiler from hoisting all NCK chunks of them into
        // registers (hundreds of VGPRs) instead of reading LDS chunk by chunk.
        int qoff = 0;
        asm volatile("" : "+v"(qoff));
        const float *qt = qrow + qoff;
        float4 rn[4];
        if constexpr (COS) load_tile_norms(rnorm, t, lane, rn);
        floatx16 acc[ACC];
#pragma unroll
        for (int h = 0; h < ACC; ++h)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[h][v] = 0.f;
#pragma unroll
        for (int j = 0; j < NCK; ++j) {
            const int s = j % KPF;
            const int jn = (j + 1 < NCK) ? j + 1 : 0;  // the next tile starts again at chunk 0
            float4 anext[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) anext[i] = *reinterpret_cast<const float4 *>(qt + jn * 32 + 4 * i);
            __builtin_amdgcn_sched_barrier(0);  // issue them before this chunk's MFMAs
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[j % ACC] = __builtin_amdgcn_mfma_f32_32x32x2f32(comp(buf[s][i], e), comp(acur[i], e),
                                                                        acc[j % ACC], 0, 0, 0);
            }
            if (j + KPF < NCK)
                load_chunk(p, j + KPF, buf[s]);
            else
                load_chunk(pn, j + KPF - NCK, buf[s]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 4; ++i) acur[i] = anext[i];
        }
#pragma unroll
        for (int h = 1; h < ACC; ++h)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[0][v] += acc[h][v];
        store_tile<COS>(acc[0], t, n, q, lane, scores, ld, tmax, tld, rn, qn);
        p = pn;
    }
}

// Inner products for a depth of exactly d = 32 NCK (NCK in {8, 12, 16, 24}),
// one wave per SIMD, with the whole query block held in registers and the
// corpus streamed into LDS by direct loads.  Each wave owns consecutive 32-row
// tiles; a tile is consumed in chunks of 32 columns (32 rows x 128 bytes = 4 KB)
// through a ring of NR chunk slots in the wave's own LDS (no barrier: only the
// wave itself writes and reads its slots).
//
//   - Loads: four direct-to-LDS instructions per chunk, each 8 rows x 128
//     contiguous bytes with the non-temporal hint; unit u of row r lands at
//     16-byte position u ^ f(r) of the row's 128-byte slot row (f below), which
//     keeps the MFMA-layout reads free of bank conflicts; loads run NR - 2
//     chunks ahead, across the wave's tiles.
//   - Operands: for an MFMA step lane (m, kk) supplies corpus row m and query m
//     at column 32 c + 4 (4 kk + i) + e of chunk c (i, e = 0..3): one 16-byte
//     LDS read of the corpus unit and the matching query float4 from registers
//     feed four v_mfma_f32_32x32x2_f32.  The next chunk's corpus operands are
//     read before the current chunk's sixteen MFMAs issue.
//   - Output: the tile's 32 x 32 sums are transposed through a 4 KB stage in
//     LDS so that each store instruction writes 8 whole 128-byte score lines
//     (non-temporal); per query the tile's maximum goes to tmax.
// The query block costs d / 2 registers per lane (384 at d = 768), which is why
// d = 1024 keeps the register-staged kernel above.  A ragged last tile is
// loaded from row n - 32 (so every load is a whole row) and only its rows from
// 32 t on are stored; n < 32 takes the other kernel.
template <int NCK>
struct DmaRing {
    static constexpr int value = (NCK % 8 == 0) ? 8 : 6;  // slots, a divisor of NCK
};

template <int NCK>
__global__ __launch_bounds__(256, 1) void mfma_scores_dma_kernel(const float *__restrict__ corpus, int64_t n,
                                                                 const float *__restrict__ queries, int q,
                                                                 float *__restrict__ scores, int64_t ld,
                                                                 float *__restrict__ tmax, int64_t tld,
                                                                 int64_t tiles_per_wave) {
    constexpr int d = NCK * 32;
    constexpr int NR = DmaRing<NCK>::value;
    static_assert(NCK % NR == 0 && NR >= 4, "a chunk's ring slot must be a compile-time constant");
    extern __shared__ __align__(16) char dma_lds[];  // per wave: NR chunk slots of 4 KB, then a 4 KB stage
    const int lane = threadIdx.x & 63;
    const int wv = wave_in_group();
    const int m = lane & 31;
    const int kk = lane >> 5;
    const int64_t wave = (int64_t)blockIdx.x * 4 + wv;
    const int64_t tiles = (n + 31) / 32;
    const int64_t t_begin = wave * tiles_per_wave;
    const int64_t t_end = (t_begin + tiles_per_wave < tiles) ? t_begin + tiles_per_wave : tiles;
    if (t_begin >= t_end) return;  // no barrier follows

    // query operand of lane (m, kk): Q[m][32 c + 4 (4 kk + i) + e], zero for m >= q
    float4 qreg[NCK][4];
#pragma unroll
    for (int c = 0; c < NCK; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            qreg[c][i] = (m < q) ? *reinterpret_cast<const float4 *>(queries + (int64_t)m * d + c * 32 + 4 * (4 * kk + i))
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
    char *const ring = dma_lds + wv * ((NR + 1) * 4096);
    char *const stage = ring + NR * 4096;
    const uint32_t ring_lds = lds_addr(ring);
    // direct-load lane mapping: instruction p of a chunk covers rows 8 p .. 8 p + 7
    int voff[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int r = 8 * p + (lane >> 3);
        const int u = (lane & 7) ^ dma_swizzle(r);
        voff[p] = (r * d + u * 4) * 4;
    }
    int roff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) roff[i] = m * 128 + (((4 * kk + i) ^ dma_swizzle(m)) << 4);
    auto load_row0 = [&](int64_t t) -> int64_t {
        const int64_t r = t * 32;
        return (r + 32 > n) ? n - 32 : r;
    };
    auto issue = [&](int64_t lr0, int c, int slot) {
        const char *base = reinterpret_cast<const char *>(corpus + lr0 * d + c * 32);
#pragma unroll
        for (int p = 0; p < 4; ++p) dma16_nt(base, voff[p], ring_lds + slot * 4096 + p * 1024);
    };
    const int64_t lr_first = load_row0(t_begin);
#pragma unroll
    for (int c = 0; c < NR - 1; ++c) issue(lr_first, c, c);
    float4 a[2][4];
    wait_vmcnt<4 * (NR - 2)>();  // chunk 0 has landed
#pragma unroll
    for (int i = 0; i < 4; ++i) a[0][i] = *reinterpret_cast<const float4 *>(ring + roff[i]);
    for (int64_t t = t_begin; t < t_end; ++t) {
        const int64_t lr = load_row0(t);
        const int64_t lr_next = (t + 1 < t_end) ? load_row0(t + 1) : lr;  // past the last tile: reload, unused
        floatx16 acc;
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
        for (int c = 0; c < NCK; ++c) {
            // chunk c + 1 (the next tile's chunk 0 after the last) must have
            // landed: the loads issued after it are chunks c + 2 .. c + NR - 2
            wait_vmcnt<4 * (NR - 3)>();
            __builtin_amdgcn_sched_barrier(0);
            {
                const char *src = ring + ((c + 1) % NR) * 4096;
#pragma unroll
                for (int i = 0; i < 4; ++i) a[(c + 1) & 1][i] = *reinterpret_cast<const float4 *>(src + roff[i]);
            }
            __builtin_amdgcn_sched_barrier(0);
            {
                // refill the slot of chunk c - 1, whose operands were read an iteration ago
                const int cn = c + NR - 1;  // a constant once the loop is unrolled
                if (cn < NCK)
                    issue(lr, cn, cn % NR);
                else
                    issue(lr_next, cn - NCK, cn % NR);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(comp(a[c & 1][i], e), comp(qreg[c][i], e), acc, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        // lane (j, h) holds rows 8 g + 4 h + c' (register 4 g + c') of query j
        const int j = lane & 31;
        const int h = lane >> 5;
        const int64_t row0 = t * 32;
        float mx = -INFINITY;
        if (lr == row0) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 v = make_float4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
                mx = fmaxf(mx, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
                const int u = 2 * g + h;  // 16-byte unit of the query's 128-byte score line
                *reinterpret_cast<float4 *>(stage + j * 128 + ((u ^ dma_swizzle(j)) << 4)) = v;
            }
            // 8 queries x 128 bytes per store instruction
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int jj = 8 * k + (lane >> 3);
                const int su = lane & 7;
                const float4 v = *reinterpret_cast<const float4 *>(stage + jj * 128 + ((su ^ dma_swizzle(jj)) << 4));
                if (jj < q) {
                    const f32x4_t w = {v.x, v.y, v.z, v.w};
                    __builtin_nontemporal_store(w, reinterpret_cast<f32x4_t *>(scores + (int64_t)jj * ld + row0 + 4 * su));
                }
            }
        } else if (j < q) {  // the ragged last tile, loaded from n - 32: rows from row0 on
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int64_t r = lr + 8 * g + 4 * h + c;
                    if (r >= row0) {
                        scores[(int64_t)j * ld + r] = acc[4 * g + c];
                        mx = fmaxf(mx, acc[4 * g + c]);
                    }
                }
        }
        mx = fmaxf(mx, __uint_as_float(xor_u32<32>(__float_as_uint(mx))));
        if (h == 0 && j < q) tmax[(int64_t)j * tld + t] = mx;
    }
    wait_vmcnt<0>();  // no direct load may still be writing LDS when the wave ends
}

static size_t dma_lds_bytes(int nck) { return (size_t)4 * ((nck % 8 == 0 ? 8 : 6) + 1) * 4096; }
#define RT_MFMA_DMA(X) X(8) X(12) X(16) X(24)

static size_t mfma_lds_bytes(int d, int kpf) { return (size_t)kMfmaMaxQ * (mfma_cols(d, kpf) + 4) * sizeof(float); }

// Depths with a compile-time kernel (d = 32 * NCK); others take the runtime loop.
#define RT_MFMA_FIXED(X) X(8) X(12) X(16) X(24) X(32)
constexpr int kFixedPrefetch = 2;
constexpr int kFixedThreads = 1024;
constexpr int kFixedAcc = 2;

template <bool COS>
static hipError_t prepare_metric() {
    hipError_t err = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&mfma_scores_kernel<kMfmaPrefetch, kMfmaThreads, kMfmaAcc, COS>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)mfma_lds_bytes(kMfmaMaxD, kMfmaPrefetch));
#define RT_PREP(NCK)                                                                                          \
    if (err == hipSuccess)                                                                                    \
        err = hipFuncSetAttribute(reinterpret_cast<const void *>(                                             \
                                      &mfma_scores_fixed_kernel<NCK, kFixedPrefetch, kFixedThreads, kFixedAcc, COS>), \
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)mfma_lds_bytes(NCK * 32, 1));
    RT_MFMA_FIXED(RT_PREP)
#undef RT_PREP
    return err;
}

hipError_t prepare_mfma_scores() {
    hipError_t err = prepare_metric<false>();
    if (err == hipSuccess) err = prepare_metric<true>();
#define RT_PREP_DMA(NCK)                                                                                 \
    if (err == hipSuccess)                                                                               \
        err = hipFuncSetAttribute(reinterpret_cast<const void *>(&mfma_scores_dma_kernel<NCK>),          \
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)dma_lds_bytes(NCK));
    RT_MFMA_DMA(RT_PREP_DMA)
#undef RT_PREP_DMA
    return err;
}

template <bool COS>
static hipError_t launch_metric(const float *corpus, int64_t n, int d, const float *queries, int q,
                                const float *rnorm, float *scores, int64_t ld, float *tmax, int64_t tld, int num_cus,
                                hipStream_t stream) {
    const int64_t tiles = (n + 31) / 32;
#define RT_FIXED(NCK)                                                                                            \
    if (d == NCK * 32) {                                                                                         \
        constexpr int w = kFixedThreads / 64;                                                                    \
        const int64_t tpw = (tiles + (int64_t)num_cus * w - 1) / ((int64_t)num_cus * w);                         \
        const int64_t blocks = (tiles + tpw * w - 1) / (tpw * w);                                                \
        hipLaunchKernelGGL((mfma_scores_fixed_kernel<NCK, kFixedPrefetch, kFixedThreads, kFixedAcc, COS>),       \
                           dim3((unsigned)blocks), dim3(kFixedThreads), mfma_lds_bytes(d, 1), stream, corpus, n, \
                           queries, q, rnorm, scores, ld, tmax, tld, tpw);                                       \
        return hipGetLastError();                                                                                \
    }
    RT_MFMA_FIXED(RT_FIXED)
#undef RT_FIXED
    constexpr int w = kMfmaThreads / 64;
    const int64_t tiles_per_wave = (tiles + (int64_t)num_cus * w - 1) / ((int64_t)num_cus * w);
    const int64_t blocks = (tiles + tiles_per_wave * w - 1) / (tiles_per_wave * w);
    hipLaunchKernelGGL((mfma_scores_kernel<kMfmaPrefetch, kMfmaThreads, kMfmaAcc, COS>), dim3((unsigned)blocks),
                       dim3(kMfmaThreads), mfma_lds_bytes(d, kMfmaPrefetch), stream, corpus, n, d, queries, q, rnorm,
                       scores, ld, tmax, tld, tiles_per_wave);
    return hipGetLastError();
}

hipError_t launch_mfma_scores(const float *corpus, int64_t n, int d, const float *queries, int q,
                              const float *rnorm, float *scores, int64_t ld, float *tmax, int64_t tld, int num_cus,
                              hipStream_t stream) {
    if (rnorm != nullptr)
        return launch_metric<true>(corpus, n, d, queries, q, rnorm, scores, ld, tmax, tld, num_cus, stream);
    if (n >= 32) {
        const int64_t tiles = (n + 31) / 32;
        const int64_t tpw = (tiles + (int64_t)num_cus * 4 - 1) / ((int64_t)num_cus * 4);
        const int64_t blocks = (tiles + tpw * 4 - 1) / (tpw * 4);
#define RT_DMA(NCK)                                                                                        \
        if (d == NCK * 32) {                                                                               \
            hipLaunchKernelGGL((mfma_scores_dma_kernel<NCK>), dim3((unsigned)blocks), dim3(256),           \
                               dma_lds_bytes(NCK), stream, corpus, n, queries, q, scores, ld, tmax, tld, tpw); \
            return hipGetLastError();                                                                      \
        }
        RT_MFMA_DMA(RT_DMA)
#undef RT_DMA
    }
    return launch_metric<false>(corpus, n, d, queries, q, nullptr, scores, ld, tmax, tld, num_cus, stream);
}

}  // namespace rt
