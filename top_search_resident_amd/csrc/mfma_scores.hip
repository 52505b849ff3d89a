// mfma_scores.hip -- batched inner products on CDNA4 matrix cores.
//
// A batch of q <= 32 queries against the resident corpus is a dense contraction
// S = Q . C^T (q x n, reduction over d).  The pages score one query at a time
// ("GPU-Resident Top-K for Agentic RAG", section 4, Step 2) and list concurrent
// queries as missing (section 9); with a batch the corpus is read from HBM once
// for all queries and the arithmetic runs on v_mfma_f32_32x32x2_f32.
//
// Tiling.  One 512-thread workgroup per CU stages the whole (zero-padded) 32 x d
// query block in LDS (row stride d + 4 floats to spread LDS banks).  Each wave
// owns tiles of 64 corpus rows and produces two 32 x 32 output tiles (queries x
// rows) that share the query operand.  For an MFMA step the query operand lane
// l holds Q[l % 32][c] and the corpus operand lane l holds C[row0 + l % 32][c],
// with the column c = c0 + 16 (l / 32) + 4 i + e for step (i, e); so per 32
// columns each lane issues four 16-byte corpus loads covering 64 contiguous
// bytes of its row, and the two lane halves cover the row's full 128 bytes.
// The next 32 columns are loaded while the current ones are multiplied.
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
    const int64_t tiles = (n + 63) / 64;
    const int64_t t_begin = wave * tiles_per_wave;
    const int64_t t_end = (t_begin + tiles_per_wave < tiles) ? t_begin + tiles_per_wave : tiles;
    const float *qrow = qs + m * dp + 16 * kk;

    for (int64_t t = t_begin; t < t_end; ++t) {
        const int64_t row0 = t * 64;
        const bool v0 = row0 + m < n;
        const bool v1 = row0 + 32 + m < n;
        const float *p0 = corpus + (row0 + m) * (int64_t)d + 16 * kk;
        const float *p1 = p0 + 32 * (int64_t)d;
        floatx16 acc0, acc1;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            acc0[v] = 0.f;
            acc1[v] = 0.f;
        }
        float4 b0[4], b1[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool okc = 16 * kk + 4 * i < d;
            b0[i] = ld4_or_zero(p0 + 4 * i, v0 && okc);
            b1[i] = ld4_or_zero(p1 + 4 * i, v1 && okc);
        }
        for (int c0 = 0; c0 < d; c0 += 32) {
            float4 c0b[4], c1b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                c0b[i] = b0[i];
                c1b[i] = b1[i];
            }
            const int cn = c0 + 32;
            if (cn < d) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool okc = cn + 16 * kk + 4 * i < d;
                    b0[i] = ld4_or_zero(p0 + cn + 4 * i, v0 && okc);
                    b1[i] = ld4_or_zero(p1 + cn + 4 * i, v1 && okc);
                }
            }
            float4 a[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = ld4_or_zero(qrow + c0 + 4 * i, c0 + 16 * kk + 4 * i < d);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(comp(a[i], e), comp(c0b[i], e), acc0, 0, 0, 0);
                    acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(comp(a[i], e), comp(c1b[i], e), acc1, 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int qi = 8 * (v >> 2) + 4 * kk + (v & 3);
            if (qi < q) {
                if (v0) scores[(int64_t)qi * ld + row0 + m] = acc0[v];
                if (v1) scores[(int64_t)qi * ld + row0 + 32 + m] = acc1[v];
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
    const int64_t tiles = (n + 63) / 64;
    const int64_t waves = (int64_t)num_cus * (kMfmaThreads / 64);
    const int64_t tiles_per_wave = (tiles + waves - 1) / waves;
    const int64_t blocks = (tiles + tiles_per_wave * (kMfmaThreads / 64) - 1) / (tiles_per_wave * (kMfmaThreads / 64));
    hipLaunchKernelGGL(mfma_scores_kernel, dim3((unsigned)blocks), dim3(kMfmaThreads), mfma_lds_bytes(d), stream,
                       corpus, n, d, queries, q, scores, ld, tiles_per_wave);
    return hipGetLastError();
}

}  // namespace rt
