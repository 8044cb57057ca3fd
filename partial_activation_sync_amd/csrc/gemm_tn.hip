// Weight-gradient GEMMs of the backward, straight from token-major operands:
//   out[m][n] = sum_k A[k][m] B[k][n]        (bf16 in, fp32 accumulation, bf16 out)
// with k running over tokens: dW1 = da^T x, dW2 = dZt^T Y, dWo = dZt^T H, the chain rule
// through "Tensor-Parallelism with Partially Synchronized Activations", App. A.2 Eq. 22
// and Eq. 24.  Both operands are stored token-major ([k][m], [k][n], rows contiguous), so
// the contraction runs across rows and no transposed copy is made.
//
// Tiles of 256 n x 256 m, 8 waves (4 x 2, 64 n x 128 m each), K stepped by 64 tokens
// through two LDS stages:
//   * each operand's [64 k][256] slice is copied to LDS by buffer loads that write LDS
//     directly, 512-byte row segments, rows padded to 576 bytes (36 16-byte slots);
//   * an MFMA fragment needs 8 consecutive k of one column; it is read with two
//     ds_read_b64_tr_b16.  Within each 16-lane group, source lane 4e + q addresses 4
//     columns of K row e and lane i receives column i's 4 values of those 4 rows.  With
//     576-byte rows the 4 rows of a group start 16 banks apart, so the reads of 32 lanes
//     (4 rows x 64 bytes) are conflict-free;
//   * a step's descriptors start at its first token and end with the operand, so token
//     rows past K read as zero: no tail code;
//   * the schedule, barrier placement and the epilogue through LDS follow the forward's
//     K1 / K2 kernel.
#include "caat_internal.h"
#include "bufload.h"

#if defined(__HIP_DEVICE_COMPILE__)
#define CAAT_UNROLL _Pragma("unroll")
#define CAAT_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)
#define CAAT_SCHED_GROUP(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)
#else
#define CAAT_UNROLL
#define CAAT_SCHED_FENCE()
#define CAAT_SCHED_GROUP(mask, n)
#endif

namespace caat {
namespace {

typedef short v4s __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int SG_MFMA = 0x008, SG_DS_READ = 0x100;
constexpr int BN = 256, BM = 256, BK = 64, WGN = 4, WGM = 2;
constexpr int NW = WGN * WGM, NTH = 64 * NW;
constexpr int PITCH = 36;                      // 16-byte slots per LDS row (32 + padding)
constexpr int OPSLOTS = BK * PITCH;            // one operand's slice
constexpr int SLOTS = 2 * OPSLOTS;             // B (n) slice first, then A (m)
constexpr int LOADS = SLOTS / NTH;             // loads per lane per stage
constexpr int OPBLK = OPSLOTS / 64;            // 64-slot blocks per operand
static_assert(SLOTS % NTH == 0 && OPSLOTS % 64 == 0, "stage must split into whole loads");

__device__ __forceinline__ bf16x4 read_tr(const uint4 *lds, int byte_off) {
    const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s *)(reinterpret_cast<const char *>(lds) + byte_off));
    return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ int xcd_tile(int b, int total) {
    const int xcd = b & 7, idx = b >> 3;
    const int q = total >> 3, r = total & 7;
    return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

__global__ __launch_bounds__(NTH) void k_gemm_tn(TnArgs a, int tilesN, int tilesM)
{
    constexpr int WN = BN / WGN, WM = BM / WGM;     // wave tile: n x m
    constexpr int IB = WN / 32, JB = WM / 32;       // 32 x 32 MFMA blocks per wave
    constexpr int NREAD = IB + JB, NMFMA = IB * JB;
    static_assert(NMFMA >= NREAD, "interleave needs at least one MFMA per fragment");

    __shared__ __attribute__((aligned(16))) uint4 L0[SLOTS];
    __shared__ __attribute__((aligned(16))) uint4 L1[SLOTS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave % WGN, wm = wave / WGN;
    const int per = tilesN * tilesM;
    const int tile = xcd_tile(blockIdx.x, gridDim.x);
    const int bt = tile / per, rem = tile - bt * per;
    const int tn = rem % tilesN, tm = rem / tilesN;
    const int n0 = tn * BN, m0 = tm * BM;
    const int M = a.M, N = a.N, K = a.K;

    const __bf16 *Ab = reinterpret_cast<const __bf16 *>(a.A) + (size_t)bt * a.a_stride;
    const __bf16 *Bb = reinterpret_cast<const __bf16 *>(a.B) + (size_t)bt * a.b_stride;

    // Load i of a lane fills LDS slot (i*NW + wave)*64 + lane; blocks [0, OPBLK) hold B,
    // the rest A.  Slot (row r, position c) of an operand holds columns 8c .. 8c + 7 of
    // token row r (c < 32; positions 32-35 pad the row and read as zero).
    uint32_t off[LOADS];
    CAAT_UNROLL for (int i = 0; i < LOADS; ++i) {
        const int blk = i * NW + wave;
        const bool isA = blk >= OPBLK;
        const int so = (blk - (isA ? OPBLK : 0)) * 64 + lane;
        const int r = so / PITCH, c = so % PITCH;
        const int col = (isA ? m0 : n0) + c * 8;
        const bool ok = c < 32 && col < (isA ? M : N);
        off[i] = ok ? (uint32_t)((r * (isA ? a.lda : a.ldb) + col) * 2) : OOB;
    }

    f32x16 acc[IB][JB];
    CAAT_UNROLL for (int i = 0; i < IB; ++i)
        CAAT_UNROLL for (int j = 0; j < JB; ++j)
            CAAT_UNROLL for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // Fragment addresses (bytes within a stage): lane l of group G = l / 16 is source lane
    // s = l % 16 = 4 e + q: K row 8 (G / 2) + e of the sub-step, columns 16 (G % 2) + 4 q
    // of the 32-column block; the second read of a fragment is 4 rows further.
    const int G = lane >> 4, e = (lane >> 2) & 3, q = lane & 3;
    const int rbase = (8 * (G >> 1) + e) * PITCH * 16 + (16 * (G & 1) + 4 * q) * 2;
    const int boff = rbase + (wn * WN) * 2;                      // B (n) operand
    const int aoff = OPSLOTS * 16 + rbase + (wm * WM) * 2;       // A (m) operand

    const int nsteps = (K + BK - 1) / BK;

    // The descriptors of step ks start at its first token row.
#define CAAT_ISSUE(ks, Lb)                                                                 \
    do {                                                                                   \
        const int k0_ = (ks) * BK;                                                         \
        const int left_ = K - k0_;                                                         \
        const __amdgpu_buffer_rsrc_t rB_ = make_rsrc(                                      \
            Bb + (size_t)k0_ * a.ldb, left_ > 0 ? (uint32_t)left_ * (uint32_t)a.ldb * 2u : 0u); \
        const __amdgpu_buffer_rsrc_t rA_ = make_rsrc(                                      \
            Ab + (size_t)k0_ * a.lda, left_ > 0 ? (uint32_t)left_ * (uint32_t)a.lda * 2u : 0u); \
        CAAT_UNROLL for (int i = 0; i < LOADS; ++i)                                        \
            load_lds16((i * NW + wave) >= OPBLK ? rA_ : rB_, (Lb) + (i * NW + wave) * 64,  \
                       off[i], 0);                                                         \
        CAAT_SCHED_FENCE();                                                                \
    } while (0)

    bf16x8 af[2][IB], bfr[2][JB];
#define CAAT_FRAG(Lb, byte)                                                                \
    __builtin_shufflevector(read_tr((Lb), (byte)), read_tr((Lb), (byte) + 4 * PITCH * 16), \
                            0, 1, 2, 3, 4, 5, 6, 7)
#define CAAT_READ(qq, Lb, kk)                                                              \
    do {                                                                                   \
        CAAT_UNROLL for (int i = 0; i < IB; ++i)                                           \
            af[qq][i] = CAAT_FRAG(Lb, boff + (kk) * 16 * PITCH * 16 + i * 64);             \
        CAAT_UNROLL for (int j = 0; j < JB; ++j)                                           \
            bfr[qq][j] = CAAT_FRAG(Lb, aoff + (kk) * 16 * PITCH * 16 + j * 64);            \
    } while (0)
#define CAAT_MMA(qq, i0, i1)                                                               \
    do {                                                                                   \
        CAAT_UNROLL for (int i = (i0); i < (i1); ++i)                                      \
            CAAT_UNROLL for (int j = 0; j < JB; ++j)                                       \
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                       \
                    af[qq][i], bfr[qq][j], acc[i][j], 0, 0, 0);                            \
    } while (0)
    // nm MFMAs with the NREAD fragments' reads (two each) interleaved, then a fence.
#define CAAT_INTERLEAVE(nm)                                                                \
    do {                                                                                   \
        CAAT_UNROLL for (int r = 0; r < NREAD; ++r) {                                      \
            if (r < (nm)) CAAT_SCHED_GROUP(SG_MFMA, 1);                                    \
            CAAT_SCHED_GROUP(SG_DS_READ, 2);                                               \
        }                                                                                  \
        if ((nm) > NREAD) CAAT_SCHED_GROUP(SG_MFMA, (nm) - NREAD);                         \
        CAAT_SCHED_FENCE();                                                                \
    } while (0)
#define CAAT_STEP_MORE(ks, Lb, Ln)                                                         \
    do {                                                                                   \
        CAAT_ISSUE(min((ks) + 1, nsteps - 1), Ln);                                         \
        CAAT_READ(1, Lb, 1); CAAT_MMA(0, 0, IB); CAAT_INTERLEAVE(NMFMA);                   \
        CAAT_READ(0, Lb, 2); CAAT_MMA(1, 0, IB); CAAT_INTERLEAVE(NMFMA);                   \
        CAAT_READ(1, Lb, 3); CAAT_MMA(0, 0, IB); CAAT_INTERLEAVE(NMFMA);                   \
        CAAT_MMA(1, 0, IB);                                                                \
        CAAT_SCHED_FENCE();                                                                \
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");                        \
        __builtin_amdgcn_s_barrier();                                                      \
        CAAT_SCHED_FENCE();                                                                \
        CAAT_READ(0, Ln, 0);                                                               \
    } while (0)
#define CAAT_STEP_LAST(Lb)                                                                 \
    do {                                                                                   \
        CAAT_READ(1, Lb, 1); CAAT_MMA(0, 0, IB); CAAT_INTERLEAVE(NMFMA);                   \
        CAAT_READ(0, Lb, 2); CAAT_MMA(1, 0, IB); CAAT_INTERLEAVE(NMFMA);                   \
        CAAT_READ(1, Lb, 3); CAAT_MMA(0, 0, IB); CAAT_INTERLEAVE(NMFMA);                   \
        CAAT_MMA(1, 0, IB);                                                                \
    } while (0)

    CAAT_ISSUE(0, L0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    CAAT_READ(0, L0, 0);
    // Whole pairs of steps, the load index clamped at the last step (a repeated load that
    // nothing reads), then an odd last step: as in the forward's kernel, this keeps the
    // accumulators on two paths to the epilogue.
    int kt = 0;
    for (; kt + 2 <= nsteps; kt += 2) {
        CAAT_STEP_MORE(kt, L0, L1);
        CAAT_STEP_MORE(kt + 1, L1, L0);
    }
    if (kt < nsteps) CAAT_STEP_LAST(L0);
#undef CAAT_FRAG
#undef CAAT_READ
#undef CAAT_MMA
#undef CAAT_INTERLEAVE
#undef CAAT_STEP_MORE
#undef CAAT_STEP_LAST
#undef CAAT_ISSUE

    // Epilogue through LDS.  Accumulator element v of block (i, j) in lane l is n row
    // 8 (v / 4) + 4 (l / 32) + v % 4 and m column l % 32 of that block.  The waves write
    // a [m][n] image of the tile (bf16) into the idle stages, the first 128 m rows in L0
    // and the rest in L1, 16-byte chunk C of image row r at C ^ (r & 15) with its 8-byte
    // halves swapped when bit 4 of r is set (conflict-free both ways), then every thread
    // stores whole 16-byte chunks of output rows.
    constexpr int CPR = BN / 8;
    static_assert((BM / 2) * CPR <= SLOTS && (BM * CPR) % NTH == 0, "output image");
    const int r32 = lane & 31, kh = lane >> 5;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    CAAT_UNROLL for (int j = 0; j < JB; ++j) {
        const int mb = wm * WM + j * 32;
        uint2 *img = reinterpret_cast<uint2 *>(mb < BM / 2 ? L0 : L1);
        const int r = mb % (BM / 2) + r32;
        const int sw = r & 15, hs = (r >> 4) & 1;
        CAAT_UNROLL for (int i = 0; i < IB; ++i) {
            const int cb = (wn * WN + i * 32) / 8;
            CAAT_UNROLL for (int g = 0; g < 4; ++g) {
                bf16x4 o;
                CAAT_UNROLL for (int v = 0; v < 4; ++v) o[v] = static_cast<__bf16>(acc[i][j][4 * g + v]);
                img[(r * CPR + ((cb + g) ^ sw)) * 2 + (kh ^ hs)] = __builtin_bit_cast(uint2, o);
            }
        }
    }
    __syncthreads();
    __bf16 *O = reinterpret_cast<__bf16 *>(a.out) + (size_t)bt * a.o_stride;
    CAAT_UNROLL for (int it = 0; it < BM * CPR / NTH; ++it) {
        const int qq = it * NTH + tid;
        const int row = qq / CPR, c = qq % CPR;
        const int r = row % (BM / 2);
        uint4 v = (row < BM / 2 ? L0 : L1)[r * CPR + (c ^ (r & 15))];
        if ((r >> 4) & 1) v = make_uint4(v.z, v.w, v.x, v.y);
        const int m = m0 + row, n = n0 + c * 8;
        if (m < M && n < N)
            *reinterpret_cast<uint4 *>(O + (size_t)m * a.ldo + n) = v;
    }
}

}  // namespace

bool gemm_tn_supported(const TnArgs &a) {
    // 32-bit byte offsets below the OOB marker within each operand and batch; 16-byte
    // chunks of whole rows.
    const uint64_t aspan = (uint64_t)a.K * a.lda * 2u, bspan = (uint64_t)a.K * a.ldb * 2u;
    return a.P >= 1 && a.M >= 1 && a.N >= 1 && a.K >= 1 && aspan < OOB && bspan < OOB &&
           a.M % 8 == 0 && a.N % 8 == 0 && a.lda % 8 == 0 && a.ldb % 8 == 0 && a.ldo % 8 == 0 &&
           a.lda >= a.M && a.ldb >= a.N && a.ldo >= a.N;
}

hipError_t gemm_tn_bf16(const TnArgs &a, hipStream_t s) {
    const int tilesN = (a.N + BN - 1) / BN, tilesM = (a.M + BM - 1) / BM;
    const dim3 grid(a.P * tilesN * tilesM), block(NTH);
    hipLaunchKernelGGL(k_gemm_tn, grid, block, 0, s, a, tilesN, tilesM);
    return hipGetLastError();
}

}  // namespace caat
