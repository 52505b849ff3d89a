// mfma_scores.hip -- batched inner products on CDNA4 matrix cores.
//
// A batch of q <= 32 queries against the resident corpus is a dense contraction
// S = Q . C^T (q x n, reduction over d).  The pages score one query at a time
// ("GPU-Resident Top-K for Agentic RAG", section 4, Step 2) and list concurrent
// queries as missing (section 9); with a batch the corpus is read from HBM once
// for all queries and the arithmetic runs on v_mfma_f32_32x32x2_f32.
//
// Tiling.  One workgroup of kMfmaThreads per CU stages the whole (zero-padded)
// 32 x d query block in LDS (row stride d + 4 floats to spread LDS banks).  Each
// wave owns tiles of 32 corpus rows and produces one 32 x 32 output tile
// (queries x rows) with v_mfma_f32_32x32x2_f32.  For an MFMA step the query
// operand lane l holds Q[l % 32][c] and the corpus operand lane l holds
// C[row0 + l % 32][c], with the column c = c0 + 16 (l / 32) + 4 i + e for step
// (i, e); so per 32 columns each lane issues four 16-byte corpus loads covering
// 64 contiguous bytes of its row, and the two lane halves cover the row's full
// 128-byte line.  Loads run two 32-column chunks ahead of the multiplies.  The
// loads are ordinary (cached): a line is consumed by four successive load
// instructions, and the non-temporal hint made it miss again (measured 1.7x
// slower on MI355X).
// Output element (query, row) of a 32x32 tile sits in lane row % 32 + 32 *
// ((query / 4) % 2), register (query % 4) + 4 * (query / 8); rows are stored
// contiguously per query (S row stride ld), so each store is 128 B per half-wave.
#include "kernels.hpp"

namespace rt {

typedef float floatx16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float4 ld4_or_zero(const float *p, bool ok) {
    return ok ? *reinterpret_cast<const float4 *>(p) : make_float4(0.f, 0.f, 0.f, 0.f);
}

__device__ __forceinline__ float comp(const float4 &v, int e) {
    return e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w));
}

constexpr int kPrefetch = 2;  // 32-column chunks loaded ahead of the multiplies

__global__ __launch_bounds__(kMfmaThreads) void mfma_scores_kernel(
    const float *__restrict__ corpus, int64_t n, int d, const float *__restrict__ queries, int q,
    float *__restrict__ scores, int64_t ld, int64_t tiles_per_wave) {
    extern __shared__ float qs[];
    const int dp = d + 4;
    for (int i = threadIdx.x; i < kMfmaMaxQ * d; i += blockDim.x) {
        const int r = i / d, c = i - r * d;
        qs[r * dp + c] = (r < q) ? queries[(int64_t)r * d + c] : 0.f;
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int m = lane & 31;
    const int kk = lane >> 5;
    const int64_t wave = (int64_t)blockIdx.x * (kMfmaThreads / 64) + wv;
    const int64_t tiles = (n + 31) / 32;
    const int64_t t_begin = wave * tiles_per_wave;
    const int64_t t_end = (t_begin + tiles_per_wave < tiles) ? t_begin + tiles_per_wave : tiles;
    const float *qrow = qs + m * dp + 16 * kk;
    const int nchunks = (d + 31) / 32;

    for (int64_t t = t_begin; t < t_end; ++t) {
        const int64_t row0 = t * 32;
        const bool valid = row0 + m < n;
        // rows past the end load the last row (their outputs are not stored)
        const float *p = corpus + (valid ? row0 + m : n - 1) * (int64_t)d + 16 * kk;
        floatx16 acc;
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] = 0.f;
        float4 buf[kPrefetch][4];
#pragma unroll
        for (int s = 0; s < kPrefetch; ++s) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int col = s * 32 + 16 * kk + 4 * i;
                buf[s][i] = ld4_or_zero(p + s * 32 + 4 * i, s < nchunks && col < d);
            }
        }
        for (int ci = 0; ci < nchunks; ci += kPrefetch) {
#pragma unroll
            for (int s = 0; s < kPrefetch; ++s) {
                const int chunk = ci + s;
                if (chunk < nchunks) {
                    const int c0 = chunk * 32;
                    float4 cur[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) cur[i] = buf[s][i];
                    const int cn = c0 + kPrefetch * 32;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        buf[s][i] = ld4_or_zero(p + cn + 4 * i, chunk + kPrefetch < nchunks && cn + 16 * kk + 4 * i < d);
                    float4 a[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) a[i] = ld4_or_zero(qrow + c0 + 4 * i, c0 + 16 * kk + 4 * i < d);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(comp(a[i], e), comp(cur[i], e), acc, 0, 0, 0);
                    }
                }
            }
        }
        if (valid) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int qi = 8 * (v >> 2) + 4 * kk + (v & 3);
                if (qi < q) scores[(int64_t)qi * ld + row0 + m] = acc[v];
            }
        }
    }
}

static size_t mfma_lds_bytes(int d) { return (size_t)kMfmaMaxQ * (d + 4) * sizeof(float); }

hipError_t prepare_mfma_scores() {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&mfma_scores_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)mfma_lds_bytes(kMfmaMaxD));
}

hipError_t launch_mfma_scores(const float *corpus, int64_t n, int d, const float *queries, int q, float *scores,
                              int64_t ld, int num_cus, hipStream_t stream) {
    const int64_t tiles = (n + 31) / 32;
    const int64_t waves = (int64_t)num_cus * (kMfmaThreads / 64);
    const int64_t tiles_per_wave = (tiles + waves - 1) / waves;
    const int64_t blocks = (tiles + tiles_per_wave * (kMfmaThreads / 64) - 1) / (tiles_per_wave * (kMfmaThreads / 64));
    hipLaunchKernelGGL(mfma_scores_kernel, dim3((unsigned)blocks), dim3(kMfmaThreads), mfma_lds_bytes(d), stream,
                       corpus, n, d, queries, q, scores, ld, tiles_per_wave);
    return hipGetLastError();
}

}  // namespace rt
