// cosine_math.hpp -- the cosine score and the filtered search's cosine bounds,
// shared by the device kernels and by a host export (rt_filter_cosine_bounds)
// that tests the very same code on the CPU.
//
// Range: the score is computed in fp32 from the scan's fp32 inner product acc
// and the fp32 product den = |q| |x| of the two norms.  It is meaningful while
// the elementwise products and acc are normal fp32 numbers; a row and query
// whose den underflows to 0 (|q| |x| below ~1e-45) score -inf like a zero row,
// and values whose fp32 inner product overflows are outside the input range
// (like NaN inputs).
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>

namespace rt {

// Cosine score from an inner product: acc / (|q| |x|), or -inf when that
// product of norms is not positive (a zero row or a zero query) -- the pages'
// cosine branch of the scoring kernel, in fp32 ("GPU-Resident Top-K for Agentic
// RAG", section 4, Step 2).
__host__ __device__ inline float cosine_of(float acc, float qnorm, float rnorm) {
    const float den = qnorm * rnorm;
    return den > 0.f ? acc / den : -INFINITY;
}

// Cosine bounds from the inner-product bounds a - e <= acc <= a + e of the
// plain scan's fp32 sum acc.  The plain cosine is acc / den with den = |q| |x|
// rounded to fp32 as cosine_of computes it (the same two fp32 values here, so
// the same den), or -inf when den is not positive.  Its division rounds by at
// most 2^-24 relative (2^-149 absolute below the normal range), as do a + e,
// a - e and the divisions below: widening by 2^-20 relative and FLT_MIN
// absolute covers them.  `known` false (an overflowed sum or bound) leaves the
// row's bounds at (+inf, -inf) unless den says -inf exactly, and a quotient
// that overflows gives the infinite bound on its side (never inf - inf).
__host__ __device__ inline void cosine_bounds(bool known, float a, float e, float qnorm, float rn, float &hi,
                                              float &lo) {
    const float den = qnorm * rn;
    if (!(den > 0.f)) {
        hi = -INFINITY;
        lo = -INFINITY;
        return;
    }
    if (!known) return;
    const float h = (a + e) / den;
    const float l = (a - e) / den;
    hi = fabsf(h) <= __FLT_MAX__ ? h + fmaf(fabsf(h), 0x1p-20f, __FLT_MIN__) : INFINITY;
    lo = fabsf(l) <= __FLT_MAX__ ? l - fmaf(fabsf(l), 0x1p-20f, __FLT_MIN__) : -INFINITY;
}

}  // namespace rt
