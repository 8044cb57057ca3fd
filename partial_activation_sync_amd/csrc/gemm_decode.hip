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
// up rows) and its KS waves split K.  The KS partial accumulators are summed through
// LDS in a fixed order, then the epilogue (GeLU / SwiGLU / plain store) runs in wave 0.
// Tokens beyond T and the K tail read as zero through the buffer range check.
#include "caat_internal.h"
#include "act.h"
#include "bufload.h"

#if defined(__HIP_DEVICE_COMPILE__)
#define CAAT_UNROLL _Pragma("unroll")
// Keeps the scheduler from moving instructions across this point.
#define CAAT_FENCE() __builtin_amdgcn_sched_barrier(0)
#else
#define CAAT_UNROLL
#define CAAT_FENCE()
#endif

namespace caat {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int KSTEP = 32;   // K per MFMA


// The weight copy of load_lds16 with the nontemporal hint (buffer_load ... nt lds): a
// decode step reads each weight once, so the stream need not stay in the caches.  On the
// 7B decode pair it took the replayed step from 67.4 to 63.5 µs at T = 1, 73.2 to 67.3 µs
// at T = 8 and 123.5 to 120.3 µs at T = 64.
__device__ __forceinline__ void load_lds16_stream(__amdgpu_buffer_rsrc_t r, uint4 *lds,
                                                  uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void *)lds, 16, voff, soff, 0, 2 /* nt */);
}

// Weight stream through wave-private LDS.  A wave's weight rows are copied into its own
// LDS region with buffer loads that write LDS directly, each instruction reading 1 KB of
// contiguous weights (4 rows x 256 B: 64 lanes x 16 B), in stages of KST = 128 K values;
// MFMA fragments are then read from LDS.  The global side picks, for LDS slot (row, j),
// the chunk j ^ (row % 16), so the fragment reads (16 rows at one chunk) hit 16 distinct
// bank groups.  Every wave reads only the rows it loaded itself, so no workgroup barrier
// is needed in the K loop; the two stages live in two LDS arrays so the compiler's
// per-wave wait before a fragment read covers the stage being read and leaves the next
// stage's loads in flight.  The JB token blocks (16 tokens each) are read from memory
// (they are small and stay in the caches) and each weight fragment feeds JB MFMAs.
template <int EPI, int RB, int JB, int KS>
__global__ __launch_bounds__(64 * KS) void k_gemm_decode_lds(GemmArgs a, int blocksN)
{
    constexpr int NA = (EPI == EPI_SWIGLU) ? 2 * RB : RB;
    constexpr int ROWS = NA * 16;
    constexpr int KST = 128, CH = KST / 8;          // K values and 16-byte chunks per stage
    constexpr int DMAS = ROWS * CH / 64;            // LDS-load instructions per stage
    static_assert(JB <= 4, "the KS x NA x JB reduction tiles must fit in one stage array");
    __shared__ __attribute__((aligned(16))) uint4 L0[KS][ROWS * CH];
    __shared__ __attribute__((aligned(16))) uint4 L1[KS][ROWS * CH];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int m = blockIdx.x / blocksN;
    const int n0 = (blockIdx.x - m * blocksN) * 16 * RB;
    const int N = a.N, T = a.T, K = a.K;

    const __bf16 *Wm = reinterpret_cast<const __bf16 *>(a.W) + (size_t)m * a.w_stride;
    const __bf16 *Xm = reinterpret_cast<const __bf16 *>(a.X) + (size_t)m * a.x_stride;
    const int wrows = (EPI == EPI_SWIGLU) ? a.up_off + N : N;
    const __amdgpu_buffer_rsrc_t rW =
        make_rsrc(Wm, (uint32_t)(((size_t)(a.kseg - 1) * a.w_kseg + (size_t)wrows * K) * 2u));
    const __amdgpu_buffer_rsrc_t rX =
        make_rsrc(Xm, (uint32_t)(((size_t)(a.kseg - 1) * a.x_kseg + (size_t)T * K) * 2u));

    // LDS-load d of a stage covers local rows 4d .. 4d+3; lane i fills slot (row, i % 16)
    // with global chunk (i % 16) ^ (row % 16) of that row.
    uint32_t roff[DMAS];
    int rchunk[DMAS];
    CAAT_UNROLL for (int d = 0; d < DMAS; ++d) {
        const int row = 4 * d + (lane >> 4);           // local row: block row / 16, r = row % 16
        const int blk = row >> 4, r = row & 15;
        const int n = n0 + 16 * (blk % RB) + r;
        const int grow = (blk >= RB) ? a.up_off + n : n;
        rchunk[d] = (lane & 15) ^ r;
        roff[d] = (n < N) ? ((uint32_t)grow * K + rchunk[d] * 8) * 2u : OOB;
    }
    // Token fragments straight from memory: lane l holds token 16 j + l % 16, K chunk l / 16.
    const int r16 = lane & 15, kq = (lane >> 4) * 8;
    uint32_t boff[JB];
    CAAT_UNROLL for (int j = 0; j < JB; ++j) {
        const int t = 16 * j + r16;
        boff[j] = (t < T) ? ((uint32_t)t * K + kq) * 2u : OOB;
    }

    // This wave's stages (segment st / kst, K offset (st % kst) * KST).
    const int kst = (K + KST - 1) / KST;
    const int nst = a.kseg * kst;
    const int per = (nst + KS - 1) / KS;
    const int s0 = wave * per, s1 = min(nst, s0 + per);

    f32x4 acc[NA][JB];
    CAAT_UNROLL for (int i = 0; i < NA; ++i)
        CAAT_UNROLL for (int j = 0; j < JB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Loads of stage st: its token fragments into registers, then its weights into LDS.
    // Everything stage st needs is issued before anything of stage st + 1, so the wait
    // before computing stage st (loads return in order) leaves stage st + 1 in flight.
    typedef bf16x8 XFrag[KST / 32][JB];
    auto issue = [&](int st, uint4 *Lw, XFrag &xb) {
        const int g = st / kst, k0 = (st - g * kst) * KST;
        const uint32_t sx = (uint32_t)((g * a.x_kseg + k0) * 2u);
        CAAT_UNROLL for (int u = 0; u < KST / 32; ++u)
            CAAT_UNROLL for (int j = 0; j < JB; ++j)
                xb[u][j] = load16(rX, (k0 + u * 32 + kq < K) ? boff[j] + sx + u * 64u : OOB);
        const uint32_t so = (uint32_t)((g * a.w_kseg + k0) * 2u);
        CAAT_UNROLL for (int d = 0; d < DMAS; ++d) {
            const uint32_t o = (k0 + rchunk[d] * 8 < K) ? roff[d] : OOB;
            load_lds16_stream(rW, Lw + d * 64, o, so);
        }
    };
    auto compute = [&](const uint4 *Lw, const XFrag &xb) {
        CAAT_UNROLL for (int u = 0; u < KST / 32; ++u) {
            const int c = u * 4 + (lane >> 4);          // logical chunk of this step
            CAAT_UNROLL for (int i = 0; i < NA; ++i) {
                const bf16x8 af = __builtin_bit_cast(bf16x8, Lw[(i * 16 + r16) * CH + (c ^ r16)]);
                CAAT_UNROLL for (int j = 0; j < JB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, xb[u][j], acc[i][j], 0, 0, 0);
            }
        }
    };

    // The loop body issues unconditionally (a branch around loads would make the
    // compiler wait for all of them where the paths join); the last one or two stages
    // are finished after it.
    uint4 *W0 = L0[wave], *W1 = L1[wave];
    XFrag x0, x1;
    if (s0 < s1) issue(s0, W0, x0);
    int st = s0;
    // Each issue is fenced, so the fragment reads of the stage being computed stay
    // behind the loads of the next stage.
    for (; st + 3 <= s1; st += 2) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // stage-1 reads done
        issue(st + 1, W1, x1);
        CAAT_FENCE();
        compute(W0, x0);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // stage-0 reads done
        issue(st + 2, W0, x0);
        CAAT_FENCE();
        compute(W1, x1);
    }
    if (st + 2 == s1) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        issue(st + 1, W1, x1);
        CAAT_FENCE();
        compute(W0, x0);
        compute(W1, x1);
    } else if (st + 1 == s1) {
        compute(W0, x0);
    }

    // Sum the KS partial accumulators through LDS (stage-0 array reused), fixed order.
    f32x4 *red = reinterpret_cast<f32x4 *>(&L0[0][0]);
    __syncthreads();
    if (KS > 1) {
        CAAT_UNROLL for (int i = 0; i < NA; ++i)
            CAAT_UNROLL for (int j = 0; j < JB; ++j)
                red[((wave * NA + i) * JB + j) * 64 + lane] = acc[i][j];
        __syncthreads();
        if (wave != 0) return;
        CAAT_UNROLL for (int i = 0; i < NA; ++i)
            CAAT_UNROLL for (int j = 0; j < JB; ++j) {
                f32x4 v = red[(i * JB + j) * 64 + lane];
                CAAT_UNROLL for (int w = 1; w < KS; ++w) v += red[((w * NA + i) * JB + j) * 64 + lane];
                acc[i][j] = v;
            }
    }

    // Accumulator element v of lane l is output row 4 (l / 16) + v, token 16 j + l % 16.
    __bf16 *O = reinterpret_cast<__bf16 *>(a.out) + (size_t)m * a.o_stride;
    CAAT_UNROLL for (int rb = 0; rb < RB; ++rb) {
        const int n = n0 + 16 * rb + 4 * (lane >> 4);
        if (n >= N) continue;
        CAAT_UNROLL for (int j = 0; j < JB; ++j) {
            const int t = 16 * j + r16;
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

template <int EPI, int RB, int JB, int KS>
hipError_t launch_lds(const GemmArgs &a, hipStream_t s) {
    const int blocksN = (a.N + 16 * RB - 1) / (16 * RB);
    const dim3 grid(a.P * blocksN), block(64 * KS);
    hipLaunchKernelGGL((k_gemm_decode_lds<EPI, RB, JB, KS>), grid, block, 0, s, a, blocksN);
    return hipGetLastError();
}

// The epilogues other than SwiGLU share their launch shapes.
template <int RB, int JB, int KS>
hipError_t launch_plain(const GemmArgs &a, hipStream_t s) {
    switch (a.epi) {
    case EPI_GELU: return launch_lds<EPI_GELU, RB, JB, KS>(a, s);
    case EPI_GELU_TANH: return launch_lds<EPI_GELU_TANH, RB, JB, KS>(a, s);
    default: return launch_lds<EPI_STORE, RB, JB, KS>(a, s);
    }
}

}  // namespace

// The weight-streaming kernel wins while few tokens feed each weight row; past that the
// tiled MFMA kernel (64-token tiles, four stages) takes over.  Measured on the 7B decode
// shapes, three weight copies rotated, µs:
//   * kernels alone (weight-streaming against 64-token tiles): K2 (K = 1376) 18.9 / 18.4
//     at T = 12, 19.5 / 18.5 at T = 16; the out-projection (K = 512) 9.2 / 9.5 at T = 48,
//     10.3 / 9.7 at T = 64; K1 (SwiGLU, K = 4096) 32.3 against ~37 at T = 16;
//   * the replayed MLP step, rules compared on one box: K2 on the tiles past 8 tokens took
//     T = 12 / 16 from 58.7 / 62.1 to 57.6 / 60.2 us; K1 on the tiles past 16 tokens took
//     T = 17 / 24 / 32 / 40 / 48 from 65.8 / 66.9 / 68.9 / 71.1 / 75.3 to 61.5 / 61.9 /
//     63.3 / 65.0 / 66.8 us.
// So: long contractions past 8 tokens (16 for SwiGLU, whose weight blocks carry two rows
// per output), every GEMM past 48.
bool gemm_decode_applies(const GemmArgs &a) {
    if (a.T > 48) return false;
    if (a.K < 1024) return true;
    return a.T <= (a.epi == EPI_SWIGLU ? 16 : 8);
}

// Launch shapes, measured on the 7B decode GEMMs (three weight copies rotated so the
// weights stream from HBM; K1: SwiGLU, N = 1376 per rank, K = 4096; K2: N = 4096,
// K = 1376; out-projection: N = 4096, K = 512):
//   * few token blocks and a long K: one weight block per wave (two for SwiGLU: gate and
//     up) with K split over 4 waves, so every wave keeps two stages in flight (K1 at
//     T <= 16 and K2 at T <= 8: 28.1 and 16.3 us at T = 1);
//   * otherwise each token fragment read from L2 should feed more weight rows: for the
//     SwiGLU epilogue two blocks per wave (64 weight rows), for the plain and GeLU ones
//     four (64 rows) once T > 8 (K2 at T = 16 / 32 / 64: 21.7 / 25.8 / 34.8 -> 19.5 /
//     22.0 / 25.7 us; the out-projection at T = 64: 13.5 -> 10.3 us).
hipError_t gemm_decode_bf16(const GemmArgs &a, hipStream_t s) {
    // Only batches gemm_decode_applies admits come here (at most 48 tokens, at most 8 for
    // a plain or GeLU contraction of 1024 or more, 16 for SwiGLU), so at most three token
    // blocks, and a single one with K split over the waves.
    if (!gemm_decode_applies(a)) return hipErrorInvalidValue;
    const int jb = (a.T + 15) / 16;
    if (a.epi == EPI_SWIGLU) {
        if (a.K >= 1024) return launch_lds<EPI_SWIGLU, 1, 1, 4>(a, s);
        switch (jb) {
        case 1: return launch_lds<EPI_SWIGLU, 2, 1, 1>(a, s);
        case 2: return launch_lds<EPI_SWIGLU, 2, 2, 1>(a, s);
        default: return launch_lds<EPI_SWIGLU, 2, 3, 1>(a, s);
        }
    }
    if (a.K >= 1024) return launch_plain<1, 1, 4>(a, s);
    if (a.T <= 8) return launch_plain<2, 1, 1>(a, s);
    switch (jb) {
    case 1: return launch_plain<4, 1, 1>(a, s);
    case 2: return launch_plain<4, 2, 1>(a, s);
    default: return launch_plain<4, 3, 1>(a, s);
    }
}

}  // namespace caat
