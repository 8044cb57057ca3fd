// K1 / K2: shard-batched bf16 GEMMs on CDNA4 MFMA (v_mfma_f32_32x32x16_bf16), fp32
// accumulation, for all P emulated ranks in one launch.
//
// "Tensor-Parallelism with Partially Synchronized Activations", App. A.2, Eq. 22:
//   K1 (first sum + sigma):  Y_m[t][k]  = act( sum_j x_m[t][j] W1_m[k][j] )
//   K2 (second sum):         Zt_m[t][l] = sum_k Y_m[t][k] W2_m[l][k]
// and Eq. 24 for the attention out-projection (K2 with H_m in place of Y_m).
//
// Layout: both operands are K-contiguous ("NT").  The MFMA row operand is the weight
// (output channels n), the column operand the activations (tokens t), so each lane's
// accumulator holds 4 consecutive output channels of one token and stores 8 bytes.
//
// Workgroup: 256 threads = 4 waves in a 2 x 2 grid; a BN x BT (channels x tokens)
// tile, K stepped by 64.  Global -> registers (buffer loads; out-of-range rows and the
// K tail read as zero from the buffer descriptor's range check) -> LDS, double
// buffered with one barrier per K step; the next K step's loads are in flight while
// the MFMAs of this one run.  LDS rows are 128 B (64 bf16) split in eight 16-byte
// chunks stored at chunk ^ f(row), which keeps both the 16-byte writes and the 16-byte
// fragment reads free of bank conflicts.
//
// SwiGLU: the W1 tile interleaves 32-row blocks of gate and up rows for the same Y
// columns ([g0..31, u0..31, g32..63, u32..63, ...]), so every wave holds matching
// gate/up accumulators in the same lanes and applies silu(g) * u in registers.
#include "caat_internal.h"

namespace caat {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 64;
constexpr int NT = 256;
constexpr uint32_t OOB = 0x80000000u;  // byte offset past every buffer's range
constexpr int RSRC_WORD3 = 0x00020000;  // gfx9 buffer descriptor: 32-bit dword format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                             RSRC_WORD3);
}

// 16-byte slot of (row, chunk) in a [rows][8 chunks] LDS tile.
__device__ __forceinline__ int swz(int row, int c) {
    return row * 8 + (c ^ ((row & 7) ^ ((row >> 3) & 1)));
}

__device__ __forceinline__ float gelu_erf(float v) {
    return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f));
}
__device__ __forceinline__ float gelu_tanh(float v) {
    // tanh form of GeLU (Hendrycks and Gimpel): c = sqrt(2 / pi), cubic coefficient 0.044715
    return 0.5f * v * (1.0f + tanhf(0.79788456080286536f * (v + 0.044715f * v * v * v)));
}
__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// Block index -> tile index.  Workgroups go round-robin to the 8 XCDs; give each XCD
// one contiguous range of tiles so neighbouring tiles (which share operand rows)
// meet in the same L2.
__device__ __forceinline__ int xcd_tile(int b, int total) {
    const int xcd = b & 7, idx = b >> 3;
    const int q = total >> 3, r = total & 7;
    return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

template <int BN, int BT, int EPI>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(1, 1)))
void k_gemm_bf16(GemmArgs a, int tilesN, int tilesT)
{
    constexpr int WN = BN / 2, WT = BT / 2;     // wave tile: channels x tokens
    constexpr int IB = WN / 32, JB = WT / 32;   // 32 x 32 MFMA blocks per wave
    constexpr int WCH = BN * 8 / NT;            // W 16-byte chunks per thread per K step
    constexpr int XCH = BT * 8 / NT;
    constexpr int NCOL = (EPI == EPI_SWIGLU) ? BN / 2 : BN;  // output columns per tile
    static_assert(IB % 2 == 0 || EPI != EPI_SWIGLU, "SwiGLU pairs need an even block count");

    __shared__ __attribute__((aligned(16))) uint4 lds[2][(BN + BT) * 8];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave & 1, wt = wave >> 1;

    const int per = tilesN * tilesT;
    const int tile = xcd_tile(blockIdx.x, gridDim.x);
    const int m = tile / per;
    const int rem = tile - m * per;
    const int tn = rem % tilesN, tt = rem / tilesN;
    const int n0 = tn * NCOL, t0 = tt * BT;
    const int N = a.N, T = a.T, K = a.K;

    const __bf16 *Wm = reinterpret_cast<const __bf16 *>(a.W) + (size_t)m * a.w_stride;
    const __bf16 *Xm = reinterpret_cast<const __bf16 *>(a.X) + (size_t)m * a.x_stride;
    const int wrows = (EPI == EPI_SWIGLU) ? a.up_off + N : N;
    const __amdgpu_buffer_rsrc_t rW = make_rsrc(Wm, (uint32_t)wrows * K * 2u);
    const __amdgpu_buffer_rsrc_t rX = make_rsrc(Xm, (uint32_t)T * K * 2u);

    // Per-thread load descriptors: byte offset at k = 0 (or OOB) and LDS slot.
    uint32_t woff[WCH], xoff[XCH];
    int wslot[WCH], xslot[XCH], wk[WCH], xk[XCH];
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
        const int q = tid + i * NT, row = q >> 3, c = q & 7;
        int wrow;
        bool ok;
        if (EPI == EPI_SWIGLU) {
            const int blk = row >> 5;
            const int y = n0 + (blk >> 1) * 32 + (row & 31);
            ok = y < N;
            wrow = (blk & 1) ? a.up_off + y : y;
        } else {
            wrow = n0 + row;
            ok = wrow < N;
        }
        woff[i] = ok ? ((uint32_t)wrow * K + c * 8) * 2u : OOB;
        wk[i] = c * 8;
        wslot[i] = swz(row, c);
    }
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
        const int q = tid + i * NT, row = q >> 3, c = q & 7;
        const int t = t0 + row;
        xoff[i] = (t < T) ? ((uint32_t)t * K + c * 8) * 2u : OOB;
        xk[i] = c * 8;
        xslot[i] = BN * 8 + swz(row, c);
    }

    uint4 wreg[WCH], xreg[XCH];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < WCH; ++i) {
            const uint32_t off = (k0 + wk[i] < K) ? woff[i] + k0 * 2u : OOB;
            auto v = __builtin_amdgcn_raw_buffer_load_b128(rW, off, 0, 0);
            wreg[i] = make_uint4(v[0], v[1], v[2], v[3]);
        }
#pragma unroll
        for (int i = 0; i < XCH; ++i) {
            const uint32_t off = (k0 + xk[i] < K) ? xoff[i] + k0 * 2u : OOB;
            auto v = __builtin_amdgcn_raw_buffer_load_b128(rX, off, 0, 0);
            xreg[i] = make_uint4(v[0], v[1], v[2], v[3]);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < WCH; ++i) lds[buf][wslot[i]] = wreg[i];
#pragma unroll
        for (int i = 0; i < XCH; ++i) lds[buf][xslot[i]] = xreg[i];
    };

    f32x16 acc[IB][JB];
#pragma unroll
    for (int i = 0; i < IB; ++i)
#pragma unroll
        for (int j = 0; j < JB; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const int nk = (K + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    const int r32 = lane & 31, khalf = lane >> 5;
    for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) gload((kt + 1) * BK);
        const uint4 *L = lds[kt & 1];
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int c = kk * 2 + khalf;
            bf16x8 af[IB], bfr[JB];
#pragma unroll
            for (int i = 0; i < IB; ++i)
                af[i] = __builtin_bit_cast(bf16x8, L[swz(wn * WN + i * 32 + r32, c)]);
#pragma unroll
            for (int j = 0; j < JB; ++j)
                bfr[j] = __builtin_bit_cast(bf16x8, L[BN * 8 + swz(wt * WT + j * 32 + r32, c)]);
#pragma unroll
            for (int i = 0; i < IB; ++i)
#pragma unroll
                for (int j = 0; j < JB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) sstore((kt + 1) & 1);
        __syncthreads();
    }

    // Epilogue.  Accumulator element v of block (i, j) in lane l is channel row
    // 8 (v / 4) + 4 (l / 32) + v % 4 and token column l % 32 of that block.
    __bf16 *O = reinterpret_cast<__bf16 *>(a.out) + (size_t)m * a.o_stride;
#pragma unroll
    for (int j = 0; j < JB; ++j) {
        const int t = t0 + wt * WT + j * 32 + r32;
        if (t >= T) continue;
        __bf16 *orow = O + (size_t)t * N;
        if (EPI == EPI_SWIGLU) {
#pragma unroll
            for (int i = 0; i < IB; i += 2) {
                const int yb = n0 + ((wn * IB + i) >> 1) * 32;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int y = yb + 8 * g + 4 * khalf;
                    if (y >= N) continue;
                    bf16x4 o;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        o[q] = static_cast<__bf16>(silu(acc[i][j][4 * g + q]) * acc[i + 1][j][4 * g + q]);
                    *reinterpret_cast<bf16x4 *>(orow + y) = o;
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < IB; ++i) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int n = n0 + wn * WN + i * 32 + 8 * g + 4 * khalf;
                    if (n >= N) continue;
                    bf16x4 o;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float v = acc[i][j][4 * g + q];
                        if (EPI == EPI_GELU) v = gelu_erf(v);
                        if (EPI == EPI_GELU_TANH) v = gelu_tanh(v);
                        o[q] = static_cast<__bf16>(v);
                    }
                    *reinterpret_cast<bf16x4 *>(orow + n) = o;
                }
            }
        }
    }
}

template <int BN, int BT>
hipError_t launch(const GemmArgs &a, hipStream_t s) {
    const int ncol = (a.epi == EPI_SWIGLU) ? BN / 2 : BN;
    const int tilesN = (a.N + ncol - 1) / ncol;
    const int tilesT = (a.T + BT - 1) / BT;
    const dim3 grid(a.P * tilesN * tilesT), block(NT);
    switch (a.epi) {
    case EPI_GELU:
        hipLaunchKernelGGL((k_gemm_bf16<BN, BT, EPI_GELU>), grid, block, 0, s, a, tilesN, tilesT);
        break;
    case EPI_GELU_TANH:
        hipLaunchKernelGGL((k_gemm_bf16<BN, BT, EPI_GELU_TANH>), grid, block, 0, s, a, tilesN, tilesT);
        break;
    case EPI_SWIGLU:
        hipLaunchKernelGGL((k_gemm_bf16<BN, BT, EPI_SWIGLU>), grid, block, 0, s, a, tilesN, tilesT);
        break;
    default:
        hipLaunchKernelGGL((k_gemm_bf16<BN, BT, EPI_STORE>), grid, block, 0, s, a, tilesN, tilesT);
        break;
    }
    return hipGetLastError();
}

}  // namespace

bool gemm_bf16_supported(const GemmArgs &a) {
    // Byte offsets are 32-bit and must stay below the OOB marker.
    const uint64_t wrows = (a.epi == EPI_SWIGLU) ? (uint64_t)a.up_off + a.N : (uint64_t)a.N;
    return wrows * a.K * 2u < OOB && (uint64_t)a.T * a.K * 2u < OOB && a.K % 8 == 0 &&
           a.N % 8 == 0;
}

hipError_t gemm_bf16(const GemmArgs &a, hipStream_t s) {
    const int ncol256 = (a.epi == EPI_SWIGLU) ? 128 : 256;
    const long tiles256 = (long)a.P * ((a.N + ncol256 - 1) / ncol256) * ((a.T + 255) / 256);
    if (tiles256 >= 512) return launch<256, 256>(a, s);
    return launch<128, 128>(a, s);
}

}  // namespace caat
