// K1 / K2 in fp32 (the fp32 storage path): the same shard-batched NT GEMM as the bf16
// MFMA kernels, with the same epilogues, on plain fp32 FMAs.
//
// "Tensor-Parallelism with Partially Synchronized Activations", App. A.2, Eq. 22 / 24.
//
// The fp32 shapes are small (the P = 2, h = 256 sublayer: 16 to 32 output tiles of
// 64 x 64), so a launch has few workgroups and each walks a long contraction; a
// workgroup that steps through K alone is bound by the latency of each step's loads.
// Here the 4 waves of a workgroup split the contraction (over every K segment in turn)
// into 4 contiguous ranges and each computes the whole 64 x 64 tile over its range:
//   * per step of 16, a wave copies its X [16][64] and W [16][64] slabs (and the up rows
//     for SwiGLU) into its own LDS region and reads them back for 8 x 8 outputs per lane;
//     the next step's global loads are issued before the current step is computed;
//   * the four partial tiles are then summed through LDS in wave order (fixed, so the
//     results do not depend on timing), and the epilogue runs on the sum.
// Ragged edges read as zero and are masked on store.
#include "caat_internal.h"

namespace caat {
namespace {

constexpr int TB = 64, NB = 64, BKF = 16, NWV = 4;

template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_f32(GemmArgs a)
{
    constexpr bool GLU = EPI == EPI_SWIGLU;
    constexpr int NS = GLU ? 3 : 2;                      // slabs per step: X, W (, U)
    __shared__ float slab[NWV][NS][BKF][TB + 1];
    __shared__ float red[NWV][TB * NB];

    const int m = blockIdx.z, t0 = blockIdx.y * TB, n0 = blockIdx.x * NB;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const float *Xm = reinterpret_cast<const float *>(a.X) + (size_t)m * a.x_stride;
    const float *Wm = reinterpret_cast<const float *>(a.W) + (size_t)m * a.w_stride;
    const int N = a.N, T = a.T, K = a.K;

    // This wave's contiguous range of steps over all K segments.
    const int nk = (K + BKF - 1) / BKF;
    const int G = a.kseg * nk;
    const int S = (G + NWV - 1) / NWV;
    const int g0 = wave * S;

    // Loads of one step: 64 rows x 16 k per slab, lane l reads row l (16 consecutive k as
    // four 16-byte loads: K, the segment strides and up_off K are multiples of 8).
    float4 ld[NS][BKF / 4];
    auto issue = [&](int g) {
        const bool ok = g < G && g - g0 < S;
        const int seg = ok ? g / nk : 0;
        const int k0 = ok ? (g - seg * nk) * BKF : 0;
        const float *Xg = Xm + (size_t)seg * a.x_kseg;
        const float *Wg = Wm + (size_t)seg * a.w_kseg;
        const int t = t0 + lane, n = n0 + lane;
        const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int v = 0; v < BKF / 4; ++v) {
            const int k = k0 + 4 * v;
            const bool kin = ok && k < K;
            ld[0][v] = (kin && t < T) ? *reinterpret_cast<const float4 *>(Xg + (size_t)t * K + k) : z;
            ld[1][v] = (kin && n < N) ? *reinterpret_cast<const float4 *>(Wg + (size_t)n * K + k) : z;
            if (GLU)
                ld[NS - 1][v] = (kin && n < N)
                    ? *reinterpret_cast<const float4 *>(Wg + (size_t)(a.up_off + n) * K + k) : z;
        }
    };

    const int ty = lane >> 3, tx = lane & 7;          // tokens ty*8 + i, columns tx + 8 j
    float acc[8][8] = {}, accu[8][8] = {};   // accu: SwiGLU up rows only
    issue(g0);
    for (int s = 0; s < S; ++s) {
#pragma unroll
        for (int q = 0; q < NS; ++q)
#pragma unroll
            for (int v = 0; v < BKF / 4; ++v) {
                slab[wave][q][4 * v + 0][lane] = ld[q][v].x;
                slab[wave][q][4 * v + 1][lane] = ld[q][v].y;
                slab[wave][q][4 * v + 2][lane] = ld[q][v].z;
                slab[wave][q][4 * v + 3][lane] = ld[q][v].w;
            }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        issue(g0 + s + 1);                            // the next step flies while this one runs
#pragma unroll
        for (int kk = 0; kk < BKF; ++kk) {
            float xv[8], wv[8], uv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) xv[i] = slab[wave][0][kk][ty * 8 + i];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                wv[j] = slab[wave][1][kk][tx + 8 * j];
                if (GLU) uv[j] = slab[wave][NS - 1][kk][tx + 8 * j];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    acc[i][j] = fmaf(xv[i], wv[j], acc[i][j]);
                    if (GLU) accu[i][j] = fmaf(xv[i], uv[j], accu[i][j]);
                }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // Sum of the four partial tiles in wave order; thread t then owns outputs
    // t + 256 q (row (t + 256 q) / 64, column (t + 256 q) % 64).
    float sum[16], sumu[16];
    auto reduce = [&](float (&part)[8][8], float *out) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) red[wave][(ty * 8 + i) * NB + tx + 8 * j] = part[i][j];
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int o = threadIdx.x + 256 * q;
            float v = red[0][o];
#pragma unroll
            for (int w = 1; w < NWV; ++w) v += red[w][o];
            out[q] = v;
        }
        __syncthreads();
    };
    reduce(acc, sum);
    if (GLU) reduce(accu, sumu);

    float *O = reinterpret_cast<float *>(a.out) + (size_t)m * a.o_stride;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int o = threadIdx.x + 256 * q;
        const int t = t0 + o / NB, n = n0 + o % NB;
        if (t >= T || n >= N) continue;
        float v = sum[q];
        if (EPI == EPI_GELU) v = 0.5f * v * erfcf(-v * 0.70710678118654752f);
        if (EPI == EPI_GELU_TANH)
            v = 0.5f * v * (1.0f + tanhf(0.79788456080286536f * (v + 0.044715f * v * v * v)));
        if (EPI == EPI_SWIGLU) v = v / (1.0f + expf(-v)) * sumu[q];
        O[(size_t)t * a.ldo + n] = v;
    }
}

}  // namespace

hipError_t gemm_f32(const GemmArgs &a, hipStream_t s) {
    const dim3 grid((a.N + NB - 1) / NB, (a.T + TB - 1) / TB, a.P), block(256);
    switch (a.epi) {
    case EPI_GELU: hipLaunchKernelGGL(k_gemm_f32<EPI_GELU>, grid, block, 0, s, a); break;
    case EPI_GELU_TANH: hipLaunchKernelGGL(k_gemm_f32<EPI_GELU_TANH>, grid, block, 0, s, a); break;
    case EPI_SWIGLU: hipLaunchKernelGGL(k_gemm_f32<EPI_SWIGLU>, grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL(k_gemm_f32<EPI_STORE>, grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace caat
