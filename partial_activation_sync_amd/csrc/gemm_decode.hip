// D1 / D2: the K1 / K2 GEMMs for decode batches (T <= 64 tokens), where the weights
// are read once and dominate the bytes: a weight-streaming kernel bound by HBM.
//
// "Tensor-Parallelism with Partially Synchronized Activations", App. A.2, Eq. 22 (MLP)
// and Eq. 24 (attention out-projection): the same per-rank products as the prefill
// kernels, at a shape where every weight element is used by at most 64 tokens.
//
// MFMA v_mfma_f32_16x16x32_bf16 with the weight rows as the row operand (16 output
// channels per block) and the tokens as the column operand (16 per block, JB blocks).
// A workgroup owns 16 or 32 output columns of one rank (for SwiGLU also the matching
// up rows) and its KS waves split K; each wave streams its weight slice with buffer
// loads straight into MFMA fragments (four lanes read 64 contiguous bytes of a row per
// instruction), one batch of k-steps in flight while the previous batch is multiplied.  The activations are
// small and read through the caches.  The KS partial accumulators are summed through
// LDS in a fixed order, then the epilogue (GeLU / SwiGLU / plain store) runs in wave 0.
// Tokens beyond T and the K tail read as zero through the buffer range check.
#include "caat_internal.h"

#if defined(__HIP_DEVICE_COMPILE__)
#define CAAT_UNROLL _Pragma("unroll")
#else
#define CAAT_UNROLL
#endif

namespace caat {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t OOB = 0x80000000u;
constexpr int RSRC_WORD3 = 0x00020000;
constexpr int KSTEP = 32;   // K per MFMA

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                             RSRC_WORD3);
}
__device__ __forceinline__ bf16x8 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float gelu_erf(float v) {
    return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f));
}
__device__ __forceinline__ float gelu_tanh(float v) {
    return 0.5f * v * (1.0f + tanhf(0.79788456080286536f * (v + 0.044715f * v * v * v)));
}
__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// RB: 16-column output blocks per workgroup; NA = RB (x2 for SwiGLU: gate, up) weight
// row blocks; JB: 16-token blocks; KS: waves splitting K; U: k-steps per load batch.
// Batches are double-buffered: the loads of batch b+1 are issued before the MFMAs of
// batch b, so every wave keeps one batch of loads in flight while it computes.
template <int EPI, int RB, int JB, int KS>
__global__ __launch_bounds__(64 * KS) void k_gemm_decode(GemmArgs a, int blocksN)
{
    constexpr int NA = (EPI == EPI_SWIGLU) ? 2 * RB : RB;
    constexpr int FR = NA + JB;                        // fragments per k-step
    constexpr int U = (16 / FR) >= 4 ? 4 : (16 / FR) >= 2 ? 2 : 1;
    __shared__ f32x4 red[KS > 1 ? KS : 1][NA][JB][64];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int m = blockIdx.x / blocksN;
    const int n0 = (blockIdx.x - m * blocksN) * 16 * RB;
    const int N = a.N, T = a.T, K = a.K;

    const __bf16 *Wm = reinterpret_cast<const __bf16 *>(a.W) + (size_t)m * a.w_stride;
    const __bf16 *Xm = reinterpret_cast<const __bf16 *>(a.X) + (size_t)m * a.x_stride;
    const int wrows = (EPI == EPI_SWIGLU) ? a.up_off + N : N;
    // One descriptor spans every K segment (the emulated ranks' contractions).
    const __amdgpu_buffer_rsrc_t rW =
        make_rsrc(Wm, (uint32_t)(((size_t)(a.kseg - 1) * a.w_kseg + (size_t)wrows * K) * 2u));
    const __amdgpu_buffer_rsrc_t rX =
        make_rsrc(Xm, (uint32_t)(((size_t)(a.kseg - 1) * a.x_kseg + (size_t)T * K) * 2u));

    // Fragment rows: lane l holds row l % 16 and K values 8 (l / 16) .. + 8 of a step.
    // Weight block i covers output columns n0 + 16 (i % RB) + [0, 16); for SwiGLU the
    // blocks i >= RB are the matching up rows.
    const int r16 = lane & 15, kq = (lane >> 4) * 8;
    uint32_t aoff[NA], boff[JB];
    CAAT_UNROLL for (int i = 0; i < NA; ++i) {
        const int n = n0 + 16 * (i % RB) + r16;
        const int row = (i >= RB) ? a.up_off + n : n;
        aoff[i] = (n < N) ? ((uint32_t)row * K + kq) * 2u : OOB;
    }
    CAAT_UNROLL for (int j = 0; j < JB; ++j) {
        const int t = j * 16 + r16;
        boff[j] = (t < T) ? ((uint32_t)t * K + kq) * 2u : OOB;
    }

    // This wave's range of combined K steps (segment st / ksteps, step st % ksteps),
    // processed in batches of U steps.
    const int ksteps = (K + KSTEP - 1) / KSTEP;
    const int nsteps = a.kseg * ksteps;
    const int per = (nsteps + KS - 1) / KS;
    const int s0 = wave * per;
    const int s1 = min(nsteps, s0 + per);
    const int nb = (s1 > s0) ? (s1 - s0 + U - 1) / U : 0;

    f32x4 acc[NA][JB];
    CAAT_UNROLL for (int i = 0; i < NA; ++i)
        CAAT_UNROLL for (int j = 0; j < JB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    bf16x8 fa[2][U][NA], fb[2][U][JB];
    // Loads of batch b into buffer q.  A step past this wave's range, or a chunk past
    // K, reads as zero.
#define CAAT_DLOAD(q, b)                                                                     \
    do {                                                                                     \
        CAAT_UNROLL for (int u = 0; u < U; ++u) {                                            \
            const int st = s0 + (b) * U + u;                                                 \
            const int g = st / ksteps;                                                       \
            const int k = (st - g * ksteps) * KSTEP;                                         \
            const bool in = (st < s1) && (k + kq < K);                                       \
            const uint32_t gw = (uint32_t)((g * a.w_kseg + k) * 2u);                         \
            const uint32_t gx = (uint32_t)((g * a.x_kseg + k) * 2u);                         \
            CAAT_UNROLL for (int i = 0; i < NA; ++i)                                         \
                fa[q][u][i] = load16(rW, in ? aoff[i] + gw : OOB);                           \
            CAAT_UNROLL for (int j = 0; j < JB; ++j)                                         \
                fb[q][u][j] = load16(rX, in ? boff[j] + gx : OOB);                           \
        }                                                                                    \
    } while (0)
#define CAAT_DMMA(q)                                                                         \
    do {                                                                                     \
        CAAT_UNROLL for (int u = 0; u < U; ++u)                                              \
            CAAT_UNROLL for (int i = 0; i < NA; ++i)                                         \
                CAAT_UNROLL for (int j = 0; j < JB; ++j)                                     \
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(                     \
                        fa[q][u][i], fb[q][u][j], acc[i][j], 0, 0, 0);                       \
    } while (0)

    if (nb > 0) CAAT_DLOAD(0, 0);
    int b = 0;
    for (; b + 2 <= nb; b += 2) {
        CAAT_DLOAD(1, b + 1);
        CAAT_DMMA(0);
        if (b + 2 < nb) CAAT_DLOAD(0, b + 2);
        CAAT_DMMA(1);
    }
    if (b < nb) CAAT_DMMA(0);
#undef CAAT_DLOAD
#undef CAAT_DMMA

    if (KS > 1) {
        CAAT_UNROLL for (int i = 0; i < NA; ++i)
            CAAT_UNROLL for (int j = 0; j < JB; ++j) red[wave][i][j][lane] = acc[i][j];
        __syncthreads();
        if (wave != 0) return;
        CAAT_UNROLL for (int i = 0; i < NA; ++i)
            CAAT_UNROLL for (int j = 0; j < JB; ++j) {
                f32x4 v = red[0][i][j][lane];
                CAAT_UNROLL for (int w = 1; w < KS; ++w) v += red[w][i][j][lane];
                acc[i][j] = v;
            }
    }

    // Accumulator element v of lane l is output row 4 (l / 16) + v, token l % 16.
    __bf16 *O = reinterpret_cast<__bf16 *>(a.out) + (size_t)m * a.o_stride;
    CAAT_UNROLL for (int rb = 0; rb < RB; ++rb) {
        const int n = n0 + 16 * rb + 4 * (lane >> 4);
        if (n >= N) continue;
        CAAT_UNROLL for (int j = 0; j < JB; ++j) {
            const int t = j * 16 + r16;
            if (t >= T) continue;
            bf16x4 o;
            CAAT_UNROLL for (int q = 0; q < 4; ++q) {
                float v = acc[rb][j][q];
                if (EPI == EPI_GELU) v = gelu_erf(v);
                if (EPI == EPI_GELU_TANH) v = gelu_tanh(v);
                if (EPI == EPI_SWIGLU) v = silu(v) * acc[RB + rb][j][q];
                o[q] = static_cast<__bf16>(v);
            }
            *reinterpret_cast<bf16x4 *>(O + (size_t)t * a.ldo + n) = o;
        }
    }
}

template <int RB, int JB, int KS>
hipError_t launch(const GemmArgs &a, hipStream_t s) {
    const int blocksN = (a.N + 16 * RB - 1) / (16 * RB);
    const dim3 grid(a.P * blocksN), block(64 * KS);
    switch (a.epi) {
    case EPI_GELU:
        hipLaunchKernelGGL((k_gemm_decode<EPI_GELU, RB, JB, KS>), grid, block, 0, s, a, blocksN);
        break;
    case EPI_GELU_TANH:
        hipLaunchKernelGGL((k_gemm_decode<EPI_GELU_TANH, RB, JB, KS>), grid, block, 0, s, a, blocksN);
        break;
    case EPI_SWIGLU:
        hipLaunchKernelGGL((k_gemm_decode<EPI_SWIGLU, RB, JB, KS>), grid, block, 0, s, a, blocksN);
        break;
    default:
        hipLaunchKernelGGL((k_gemm_decode<EPI_STORE, RB, JB, KS>), grid, block, 0, s, a, blocksN);
        break;
    }
    return hipGetLastError();
}

// K is split over KS waves so that many waves per SIMD stream weights at once; 8-wave
// workgroups (at most 256 registers per lane) only for one-block workgroups.
template <int RB, int JB>
hipError_t launch_ks(const GemmArgs &a, hipStream_t s) {
    const long units = (long)a.P * ((a.N + 16 * RB - 1) / (16 * RB));
    if constexpr (RB == 1) {
        if (units < 1024) return launch<RB, JB, 8>(a, s);
    }
    if (units < 4096) return launch<RB, JB, 4>(a, s);
    return launch<RB, JB, 2>(a, s);
}

}  // namespace

bool gemm_decode_applies(const GemmArgs &a) { return a.T <= 64; }

// One 16-column block per workgroup for up to 16 tokens; two above that, so each
// activation fragment read feeds twice the weight bytes.
hipError_t gemm_decode_bf16(const GemmArgs &a, hipStream_t s) {
    if (a.T <= 16) return launch_ks<1, 1>(a, s);
    if (a.T <= 32) return launch_ks<2, 2>(a, s);
    if (a.T <= 48) return launch_ks<2, 3>(a, s);
    return launch_ks<2, 4>(a, s);
}

}  // namespace caat
