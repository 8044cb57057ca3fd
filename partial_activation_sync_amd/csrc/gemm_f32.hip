// K1 / K2 in fp32 (the fp32 storage path): the same shard-batched NT GEMM as the bf16
// MFMA kernels, with the same epilogues, on plain fp32 FMAs.
//
// "Tensor-Parallelism with Partially Synchronized Activations", App. A.2, Eq. 22 / 24.
//
// 64 tokens x 64 output columns per workgroup, K in steps of 16 through LDS (over every
// K segment in turn); thread (tx, ty) owns tokens ty*4 + i and columns tx + 16 j.
// SwiGLU keeps a gate and an up accumulator per output.  Ragged edges are masked on load (zero) and on store.
#include "caat_internal.h"

namespace caat {
namespace {

constexpr int TB = 64, BKF = 16;

template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_f32(GemmArgs a)
{
    constexpr bool GLU = EPI == EPI_SWIGLU;
    __shared__ float Xs[BKF][TB + 1];
    __shared__ float Ws[BKF][TB + 1];
    __shared__ float Us[GLU ? BKF : 1][TB + 1];

    const int m = blockIdx.z, t0 = blockIdx.y * TB, n0 = blockIdx.x * TB;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const float *Xm = reinterpret_cast<const float *>(a.X) + (size_t)m * a.x_stride;
    const float *Wm = reinterpret_cast<const float *>(a.W) + (size_t)m * a.w_stride;
    const int N = a.N, T = a.T, K = a.K;

    float acc[4][4] = {}, accu[4][4] = {};
    for (int g = 0; g < a.kseg; ++g) {
        const float *Xg = Xm + (size_t)g * a.x_kseg;
        const float *Wg = Wm + (size_t)g * a.w_kseg;
        for (int k0 = 0; k0 < K; k0 += BKF) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int idx = threadIdx.x + i * 256, r = idx >> 4, kk = idx & 15;
                const int k = k0 + kk;
                const int t = t0 + r, n = n0 + r;
                Xs[kk][r] = (t < T && k < K) ? Xg[(size_t)t * K + k] : 0.f;
                Ws[kk][r] = (n < N && k < K) ? Wg[(size_t)n * K + k] : 0.f;
                if (GLU) Us[kk][r] = (n < N && k < K) ? Wg[(size_t)(a.up_off + n) * K + k] : 0.f;
            }
            __syncthreads();
#pragma unroll
            for (int kk = 0; kk < BKF; ++kk) {
                float xv[4], wv[4], uv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) xv[i] = Xs[kk][ty * 4 + i];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    wv[j] = Ws[kk][tx + 16 * j];
                    if (GLU) uv[j] = Us[kk][tx + 16 * j];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        acc[i][j] = fmaf(xv[i], wv[j], acc[i][j]);
                        if (GLU) accu[i][j] = fmaf(xv[i], uv[j], accu[i][j]);
                    }
            }
            __syncthreads();
        }
    }

    float *O = reinterpret_cast<float *>(a.out) + (size_t)m * a.o_stride;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + ty * 4 + i;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx + 16 * j;
            if (n >= N) continue;
            float v = acc[i][j];
            if (EPI == EPI_GELU) v = 0.5f * v * erfcf(-v * 0.70710678118654752f);
            if (EPI == EPI_GELU_TANH)
                v = 0.5f * v * (1.0f + tanhf(0.79788456080286536f * (v + 0.044715f * v * v * v)));
            if (EPI == EPI_SWIGLU) v = v / (1.0f + expf(-v)) * accu[i][j];
            O[(size_t)t * a.ldo + n] = v;
        }
    }
}

}  // namespace

hipError_t gemm_f32(const GemmArgs &a, hipStream_t s) {
    const dim3 grid((a.N + TB - 1) / TB, (a.T + TB - 1) / TB, a.P), block(256);
    switch (a.epi) {
    case EPI_GELU: hipLaunchKernelGGL(k_gemm_f32<EPI_GELU>, grid, block, 0, s, a); break;
    case EPI_GELU_TANH: hipLaunchKernelGGL(k_gemm_f32<EPI_GELU_TANH>, grid, block, 0, s, a); break;
    case EPI_SWIGLU: hipLaunchKernelGGL(k_gemm_f32<EPI_SWIGLU>, grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL(k_gemm_f32<EPI_STORE>, grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace caat
