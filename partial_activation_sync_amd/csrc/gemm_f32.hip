// K1 / K2 in fp32 (the fp32 storage path): the same shard-batched NT GEMM as the bf16
// MFMA kernels, with the same epilogues, on plain fp32 FMAs.
//
// "Tensor-Parallelism with Partially Synchronized Activations", App. A.2, Eq. 22 / 24.
//
// The fp32 shapes are small (the P = 2, h = 256 sublayer: a few dozen output tiles of
// 64 x 64), so a launch has few workgroups and each walks a long contraction; a
// workgroup that steps through K alone is bound by the latency of each step's loads, and
// one lane that owns 8 x 8 outputs issues 64 FMAs per K value.  So:
//   * the NWV waves of a workgroup split the contraction (over every K segment in turn)
//     into NWV contiguous ranges and each computes the whole TB x TB tile over its range:
//     per step of 16, a wave copies its X [16][TB] and W [16][TB] slabs (and the up rows
//     for SwiGLU) into its own LDS region and reads them back for its lane's outputs; the
//     next step's global loads are issued before the current step is computed;
//   * the NWV partial tiles are then summed through LDS in wave order (fixed, so the
//     results do not depend on timing), and the epilogue runs on the sum;
//   * a launch with fewer 64 x 64 tiles than compute units takes 32 x 32 or 16 x 16 tiles
//     with 8 waves instead (4 x 4 or 2 x 2 outputs per lane, twice the K split): the tiny
//     sublayer's two GEMMs, 32 and 16 workgroups of 64 x 64, become 512 and 256.
// Ragged edges read as zero (loads of past-the-edge elements are redirected and their
// values zeroed) and are masked on store.
#include "caat_internal.h"

namespace caat {
namespace {

constexpr int BKF = 16;

template <int EPI, int TB, int NWV>
__global__ __launch_bounds__(64 * NWV) void k_gemm_f32(GemmArgs a)
{
    constexpr int NB = TB;                               // square tiles
    constexpr bool GLU = EPI == EPI_SWIGLU;
    constexpr int NS = GLU ? 3 : 2;                      // slabs per step: X, W (, U)
    constexpr int LPS = TB / 16;                         // 16-byte loads per lane and slab
    constexpr int OI = TB / 8, OJ = NB / 8;              // outputs per lane: OI tokens x OJ columns
    constexpr int OQ = (TB * NB + 64 * NWV - 1) / (64 * NWV);   // summed outputs per thread
    static_assert(TB == 16 || TB == 32 || TB == 64, "tile");
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

    // Loads of one step: TB rows x 16 k per slab; lane l reads row l % TB, LPS consecutive
    // 4-k groups from group (l / TB) LPS on (16-byte loads: K, the segment strides and
    // up_off K are multiples of 8).  The loads of step s go to register set s % D, and
    // those of step s + D are issued as soon as step s has been copied to LDS, so D steps
    // are in flight while one is computed (D = 4 for the small tiles, whose short steps
    // and few steps per wave cannot cover a load's latency one step ahead).
    constexpr int D = TB <= 32 ? 4 : 1;
    const int lrow = lane % TB, lkq = (lane / TB) * LPS;
    float4 ld[D][NS][LPS];
    // A row past the matrix or a k past K loads from the operand's first element instead
    // and the value is replaced by zero, so every load is issued unconditionally (no branch
    // around it: the waits can then count the loads in flight) on 64-bit addresses.
    const int t_l = t0 + lrow, n_l = n0 + lrow;
    auto ld4 = [](const float *base, size_t idx, bool ok) {
        const uint4 u = *reinterpret_cast<const uint4 *>(base + (ok ? idx : 0));
        const uint32_t keep = ok ? 0xffffffffu : 0u;
        return make_float4(__uint_as_float(u.x & keep), __uint_as_float(u.y & keep),
                           __uint_as_float(u.z & keep), __uint_as_float(u.w & keep));
    };
    auto issue = [&](int g, float4 (&dst)[NS][LPS]) {
        const bool ok = g < G && g - g0 < S;
        const int seg = ok ? g / nk : 0;
        const int k0 = ok ? (g - seg * nk) * BKF : 0;
        const float *Xg = Xm + (size_t)seg * a.x_kseg;
        const float *Wg = Wm + (size_t)seg * a.w_kseg;
#pragma unroll
        for (int v = 0; v < LPS; ++v) {
            const int k = k0 + 4 * (lkq + v);
            const bool kin = ok && k < K;
            dst[0][v] = ld4(Xg, (size_t)t_l * K + k, kin && t_l < T);
            dst[1][v] = ld4(Wg, (size_t)n_l * K + k, kin && n_l < N);
            if (GLU) dst[NS - 1][v] = ld4(Wg, (size_t)(a.up_off + n_l) * K + k, kin && n_l < N);
        }
    };

    const int ty = lane >> 3, tx = lane & 7;          // tokens ty OI + i, columns tx + 8 j
    float acc[OI][OJ] = {}, accu[OI][OJ] = {};   // accu: SwiGLU up rows only
#pragma unroll
    for (int u = 0; u < D; ++u) issue(g0 + u, ld[u]);
    for (int sb = 0; sb < S; sb += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            if (sb + u >= S) break;
#pragma unroll
            for (int q = 0; q < NS; ++q)
#pragma unroll
                for (int v = 0; v < LPS; ++v) {
                    const int kb = 4 * (lkq + v);
                    slab[wave][q][kb + 0][lrow] = ld[u][q][v].x;
                    slab[wave][q][kb + 1][lrow] = ld[u][q][v].y;
                    slab[wave][q][kb + 2][lrow] = ld[u][q][v].z;
                    slab[wave][q][kb + 3][lrow] = ld[u][q][v].w;
                }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            issue(g0 + sb + u + D, ld[u]);                // flies while D steps are computed
#pragma unroll
            for (int kk = 0; kk < BKF; ++kk) {
                float xv[OI], wv[OJ], uv[OJ];
#pragma unroll
                for (int i = 0; i < OI; ++i) xv[i] = slab[wave][0][kk][ty * OI + i];
#pragma unroll
                for (int j = 0; j < OJ; ++j) {
                    wv[j] = slab[wave][1][kk][tx + 8 * j];
                    if (GLU) uv[j] = slab[wave][NS - 1][kk][tx + 8 * j];
                }
#pragma unroll
                for (int i = 0; i < OI; ++i)
#pragma unroll
                    for (int j = 0; j < OJ; ++j) {
                        acc[i][j] = fmaf(xv[i], wv[j], acc[i][j]);
                        if (GLU) accu[i][j] = fmaf(xv[i], uv[j], accu[i][j]);
                    }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    }

    // Sum of the NWV partial tiles in wave order; thread t then owns outputs
    // t + 64 NWV q (row (t + 64 NWV q) / NB, column (t + 64 NWV q) % NB).
    float sum[OQ], sumu[OQ];
    auto reduce = [&](float (&part)[OI][OJ], float *out) {
#pragma unroll
        for (int i = 0; i < OI; ++i)
#pragma unroll
            for (int j = 0; j < OJ; ++j) red[wave][(ty * OI + i) * NB + tx + 8 * j] = part[i][j];
        __syncthreads();
#pragma unroll
        for (int q = 0; q < OQ; ++q) {
            const int o = threadIdx.x + 64 * NWV * q;
            if (o >= TB * NB) break;
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
    for (int q = 0; q < OQ; ++q) {
        const int o = threadIdx.x + 64 * NWV * q;
        if (o >= TB * NB) break;
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

template <int TB, int NWV>
hipError_t launch_f32(const GemmArgs &a, hipStream_t s) {
    const dim3 grid((a.N + TB - 1) / TB, (a.T + TB - 1) / TB, a.P), block(64 * NWV);
    switch (a.epi) {
    case EPI_GELU: hipLaunchKernelGGL((k_gemm_f32<EPI_GELU, TB, NWV>), grid, block, 0, s, a); break;
    case EPI_GELU_TANH:
        hipLaunchKernelGGL((k_gemm_f32<EPI_GELU_TANH, TB, NWV>), grid, block, 0, s, a);
        break;
    case EPI_SWIGLU: hipLaunchKernelGGL((k_gemm_f32<EPI_SWIGLU, TB, NWV>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((k_gemm_f32<EPI_STORE, TB, NWV>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace

// The largest tile that still gives every compute unit a workgroup (the smallest when
// none does): a lane's FMAs per K value fall with the tile (64, 16, 4), and the chip's
// FMA rate needs all CUs.
hipError_t gemm_f32(const GemmArgs &a, hipStream_t s) {
    auto tiles = [&](int tb) { return (long)a.P * ((a.N + tb - 1) / tb) * ((a.T + tb - 1) / tb); };
    const long cus = 256;   // compute units of an MI355X
    if (tiles(64) >= cus) return launch_f32<64, 4>(a, s);
    if (tiles(32) >= cus) return launch_f32<32, 8>(a, s);
    return launch_f32<16, 8>(a, s);
}

}  // namespace caat
