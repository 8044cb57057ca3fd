// Activations of the bf16 forward GEMM epilogues (K1's sigma in "Tensor-Parallelism with
// Partially Synchronized Activations", App. A.2, Eq. 22).  They run once per output
// element inside the GEMMs, where the math library's branchy erff / tanhf made the GeLU
// epilogue a large share of a short-K tile; these forms are branch-free and within about
// 1.5e-6 relative of the exact function in fp32 (for |result| > 1e-3; 4e-7 absolute below
// that), far below the bf16 rounding (2^-9 relative) that follows them.
#pragma once

#include <hip/hip_runtime.h>

namespace caat {

// erfc(x) by the Chebyshev-fitted form of Press et al., Numerical Recipes (2nd ed.),
// Sec. 6.2, function erfcc: with z = |x| and t = 1 / (1 + z / 2),
//   erfc(z) = t * exp(-z^2 + c0 + t (c1 + t (c2 + ... + t c9))),
// fractional error below 1.2e-7 for every z >= 0; erfc(-z) = 2 - erfc(z).
__device__ __forceinline__ float erfc_fit(float x) {
    const float z = fabsf(x);
    const float t = __builtin_amdgcn_rcpf(1.0f + 0.5f * z);
    float q = 0.17087277f;
    q = fmaf(q, t, -0.82215223f);
    q = fmaf(q, t, 1.48851587f);
    q = fmaf(q, t, -1.13520398f);
    q = fmaf(q, t, 0.27886807f);
    q = fmaf(q, t, -0.18628806f);
    q = fmaf(q, t, 0.09678418f);
    q = fmaf(q, t, 0.37409196f);
    q = fmaf(q, t, 1.00002368f);
    q = fmaf(q, t, -1.26551223f);
    const float r = t * __expf(q - z * z);
    return x >= 0.0f ? r : 2.0f - r;
}

// GeLU, v * Phi(v) with Phi(v) = erfc(-v / sqrt 2) / 2.
__device__ __forceinline__ float gelu_erf(float v) {
    return 0.5f * v * erfc_fit(v * -0.70710678118654752f);
}

// tanh form of GeLU (Hendrycks and Gimpel): 0.5 v (1 + tanh u), u = c (v + 0.044715 v^3),
// c = sqrt(2 / pi), written as v / (1 + e^(-2u)) (the same function: 1 + tanh u =
// 2 / (1 + e^(-2u))).  For large negative v, e^(-2u) overflows to inf and the result is -0.
__device__ __forceinline__ float gelu_tanh(float v) {
    const float u2 = 1.5957691216057308f * fmaf(0.044715f * v, v * v, v);
    return v * __builtin_amdgcn_rcpf(1.0f + __expf(-u2));
}

// silu(g) = g / (1 + e^-g), the division as a hardware reciprocal (1 ulp; the result is
// rounded to bf16).
__device__ __forceinline__ float silu(float g) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

}  // namespace caat
