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
// Pipeline (BN x BT tiles, K stepped by 64; a workgroup runs a sequence of tiles):
//   * global -> LDS with buffer loads that write LDS directly (no staging registers,
//     no ds_write); rows outside the matrices and the K tail read as zero from the
//     buffer descriptor's range check;
//   * two LDS stages held in two separate arrays, so the compiler can tell the stage
//     being filled from the stage being read; one barrier per K step, after its last
//     MFMAs; the next step's loads are issued at the start of a step and fly while its
//     MFMAs run;
//   * the fragment reads for sub-step kk+1 are interleaved with the MFMAs of sub-step
//     kk; the next step's first fragments are read after the barrier, while the SIMD's
//     other wave runs its MFMAs;
//   * LDS rows are 128 B (64 bf16) split in eight 16-byte chunks stored at
//     chunk ^ f(row), which keeps the 16-byte fragment reads free of bank conflicts;
//   * the output tile is assembled in LDS stage L1 and stored in whole rows, 16 bytes
//     per lane (an activation epilogue can store the raw pre-activation too, for a
//     backward pass that then need not recompute it), while the workgroup's next tile's
//     first K step already loads into L0: the grid is at most one workgroup per
//     resident slot, so a tile's prologue latency and the workgroup launch gap hide
//     under the previous tile's epilogue (the wait for those first loads still covers
//     the previous tile's stores: vector loads and stores share one counter).
// The residual epilogues of the row GEMMs (EPI_RESID, EPI_RESID_SPLIT) read the rank's
// residual chunk where each thread stores and write R + s_priv * bf16(acc) (Eq. 9's
// r = R + Z on private channels) into the residual output instead of a partial.
// Workgroups are mapped to tiles so that each XCD (own L2) works on one contiguous
// range of tiles, which share operand rows.
//
// SwiGLU: the W1 tile interleaves 32-row blocks of gate and up rows for the same Y
// columns ([g0..31, u0..31, g32..63, u32..63, ...]), so every wave holds matching
// gate/up accumulators in the same lanes and applies silu(g) * u in registers.
#include "caat_internal.h"
#include "act.h"
#include "bufload.h"

// Scheduling directives and unroll pragmas exist only in the device pass; the host
// pass only needs the kernel's signature.
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

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 64;
constexpr int SG_MFMA = 0x008, SG_DS_READ = 0x100;


// NST: LDS stages, 2 or 4.  With 4, three K steps are in flight while one is computed
// (for the small tiles, whose short steps cannot cover a load's latency with one).
template <int BN, int BT, int WGN, int WGT, int EPI, int NST>
__global__ __launch_bounds__(64 * WGN * WGT) void k_gemm_bf16(GemmArgs a, int tilesN, int tilesT)
{
    constexpr int NW = WGN * WGT, NTH = 64 * NW;
    constexpr int WN = BN / WGN, WT = BT / WGT;     // wave tile: channels x tokens
    constexpr int IB = WN / 32, JB = WT / 32;       // 32 x 32 MFMA blocks per wave
    constexpr int SLOTS = (BN + BT) * 8;            // 16-byte LDS slots per stage
    constexpr int LOADS = SLOTS / NTH;              // loads per lane per stage
    constexpr int WLOADS = BN * 8 / NTH;            // the first WLOADS fill W rows
    constexpr int NCOL = (EPI == EPI_SWIGLU) ? BN / 2 : BN;  // output columns per tile
    constexpr int NREAD = IB + JB, NMFMA = IB * JB;
    static_assert(SLOTS % NTH == 0 && (BN * 8) % NTH == 0, "tile must split evenly");
    static_assert(EPI != EPI_SWIGLU || IB % 2 == 0, "SwiGLU pairs need an even block count");
    static_assert(NMFMA >= NREAD, "interleave needs at least one MFMA per fragment read");
    static_assert(NST == 2 || NST == 4, "two or four stages");
    static_assert(NST == 2 || LOADS % 4 == 0, "four-stage loads go out in quarters");

    __shared__ __attribute__((aligned(16))) uint4 L0[SLOTS];
    __shared__ __attribute__((aligned(16))) uint4 L1[SLOTS];
    __shared__ __attribute__((aligned(16))) uint4 L2[NST > 2 ? SLOTS : 1];
    __shared__ __attribute__((aligned(16))) uint4 L3[NST > 2 ? SLOTS : 1];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave % WGN, wt = wave / WGN;
    const int per = tilesN * tilesT, total = a.P * per;
    const int N = a.N, T = a.T, K = a.K;

    // Tiles of this workgroup.  XCD x (= block index mod 8; workgroups go round-robin to
    // the 8 XCDs, each with its own L2) owns the contiguous tile range [xs, xs + xc),
    // which shares operand rows; its nx workgroups take every nx-th tile of the range.
    // The grid never exceeds the tile count, so every workgroup has a first tile.
    const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
    const int xc = (total >> 3) + (xcd < (total & 7));
    const int xs = xcd * (total >> 3) + min(xcd, total & 7);
    const int nx = ((int)gridDim.x >> 3) + (xcd < ((int)gridDim.x & 7));
    if (idx >= xc) return;

    const int wrows = (EPI == EPI_SWIGLU) ? a.up_off + N : N;
    // One descriptor spans every K segment; a segment's offset goes in the scalar
    // offset of the load, so the per-lane offsets below stay the same for all of them.
    const int kseg = a.kseg;
    const uint32_t wbytes = (uint32_t)(((size_t)(kseg - 1) * a.w_kseg + (size_t)wrows * K) * 2u);
    const uint32_t xbytes = (uint32_t)(((size_t)(kseg - 1) * a.x_kseg + (size_t)T * K) * 2u);

    // Load i of a lane fills LDS slot (i*NW + wave)*64 + lane: a 64-slot block is 8
    // rows, row = 8 * block + lane / 8, and the slot holds chunk c = (lane & 7) ^ f(row)
    // with f(row) = (row & 7) ^ ((row >> 3) & 1) = (lane >> 3) ^ (block & 1).
    const int cl = (lane & 7) ^ ((lane >> 3) & 7);
    // Rank, first output column, first token, operand descriptors and per-lane load
    // offsets of tile TI.  The lane index passes through an empty asm so that the
    // tile-independent parts of the offsets are recomputed per tile rather than held in
    // registers across the tile loop.
#define CAAT_TILE_SETUP(TI, M, N0, T0, RW, RX, OFF)                                        \
    do {                                                                                   \
        int ln_ = lane;                                                                    \
        asm volatile("" : "+v"(ln_));                                                      \
        const int cl_ = (ln_ & 7) ^ ((ln_ >> 3) & 7);                                      \
        M = (TI) / per;                                                                    \
        const int rem_ = (TI) - M * per;                                                   \
        N0 = (rem_ % tilesN) * NCOL;                                                       \
        T0 = (rem_ / tilesN) * BT;                                                         \
        RW = make_rsrc(reinterpret_cast<const __bf16 *>(a.W) + (size_t)M * a.w_stride, wbytes); \
        RX = make_rsrc(reinterpret_cast<const __bf16 *>(a.X) + (size_t)M * a.x_stride, xbytes); \
        CAAT_UNROLL for (int i = 0; i < LOADS; ++i) {                                      \
            const int blk = i * NW + wave;                                                 \
            const int c = cl_ ^ (blk & 1);                                                 \
            const int row = blk * 8 + (ln_ >> 3);                                          \
            uint32_t grow;                                                                 \
            bool ok;                                                                       \
            if (i < WLOADS) {                                                              \
                if (EPI == EPI_SWIGLU) {                                                   \
                    const int b32 = row >> 5, y = (N0) + (b32 >> 1) * 32 + (row & 31);     \
                    ok = y < N;                                                            \
                    grow = (b32 & 1) ? a.up_off + y : y;                                   \
                } else {                                                                   \
                    grow = (N0) + row;                                                     \
                    ok = (int)grow < N;                                                    \
                }                                                                          \
            } else {                                                                       \
                grow = (T0) + row - BN;                                                    \
                ok = (int)grow < T;                                                        \
            }                                                                              \
            OFF[i] = ok ? (grow * (uint32_t)K + c * 8) * 2u : OOB;                         \
        }                                                                                  \
    } while (0)

    // Fragment slots: a wave block's rows start at a multiple of 32, so f(row) = f(r32).
    const int r32 = lane & 31, kh = lane >> 5;
    const int fr = (r32 & 7) ^ ((r32 >> 3) & 1);
    int aoff[4], boff[4];
    CAAT_UNROLL for (int kk = 0; kk < 4; ++kk) {
        aoff[kk] = (wn * WN + r32) * 8 + ((kk * 2 + kh) ^ fr);
        boff[kk] = BN * 8 + (wt * WT + r32) * 8 + ((kk * 2 + kh) ^ fr);
    }

    // The 64-token tiles serve batches of at most 64 tokens, whose GEMMs read each weight
    // once from HBM.  Each tile walks its K steps from its own starting step (tile mod
    // nsteps, wrapping round): when every workgroup reads the same K offset at once, of
    // rows a whole row apart, HBM delivered 4.4 TB/s in a probe of the bare weight stream
    // against 6.0 TB/s with staggered offsets.  The activation GEMM's weight loads also
    // carry the nontemporal hint.  7B decode K1 at T = 64: 42.1 -> 37.7 us with both; for
    // K2 (K = 1376) the hint cost 3 us and the rotation nothing, so K2 rotates only.
    constexpr bool ROTATE = BT == 64;
    constexpr bool ACT = EPI == EPI_GELU || EPI == EPI_GELU_TANH || EPI == EPI_SWIGLU;
    constexpr int WPOL = (BT == 64 && ACT) ? 2 : 0;
    const int nk = (K + BK - 1) / BK;          // K steps per segment
    const int nsteps = kseg * nk;              // K steps over all segments
    const bool ktail = (K % BK) != 0;

    // Enqueue the loads of combined K step ks of the tile with descriptors RW, RX, offsets
    // OFF and K rotation ROT into LDS stage Lb: the tile's step ks reads combined step
    // (ks + ROT) mod nsteps (segment / nk of it).  Only a ragged last step of a segment
    // masks chunks past K (they read as zero).
#define CAAT_ISSUE_T(ks, Lb, RW, RX, OFF, ROT)                                             \
    do {                                                                                   \
        int p_ = (ks);                                                                     \
        if constexpr (ROTATE) {                                                            \
            p_ += (ROT);                                                                   \
            if (p_ >= nsteps) p_ -= nsteps;                                                \
        }                                                                                  \
        const int g_ = p_ / nk;                                                            \
        const int k0_ = (p_ - g_ * nk) * BK;                                               \
        const uint32_t sw_ = (uint32_t)((g_ * a.w_kseg + k0_) * 2u);                       \
        const uint32_t sx_ = (uint32_t)((g_ * a.x_kseg + k0_) * 2u);                       \
        if (ktail && k0_ + BK > K) {                                                       \
            CAAT_UNROLL for (int i = 0; i < LOADS; ++i) {                                  \
                const int base = (i * NW + wave) * 64;                                     \
                const int c = cl ^ ((i * NW + wave) & 1);                                  \
                const uint32_t o = (k0_ + c * 8 < K) ? OFF[i] : OOB;                       \
                if (i < WLOADS) load_lds16_pol<WPOL>(RW, (Lb) + base, o, sw_);             \
                else load_lds16(RX, (Lb) + base, o, sx_);                                  \
            }                                                                              \
        } else {                                                                           \
            CAAT_UNROLL for (int i = 0; i < LOADS; ++i) {                                  \
                if (i < WLOADS) load_lds16_pol<WPOL>(RW, (Lb) + (i * NW + wave) * 64, OFF[i], sw_); \
                else load_lds16(RX, (Lb) + (i * NW + wave) * 64, OFF[i], sx_);             \
            }                                                                              \
        }                                                                                  \
        CAAT_SCHED_FENCE();                                                                \
    } while (0)
#define CAAT_ISSUE(ks, Lb) CAAT_ISSUE_T(ks, Lb, rW, rX, off, rot)
    // A quarter of step ks's loads (load indices [q LOADS / 4, (q + 1) LOADS / 4)), for
    // spreading a step's loads over the sub-steps of the step before.
#define CAAT_ISSUE_Q(ks, Lb, q)                                                            \
    do {                                                                                   \
        constexpr int Q0_ = (q) * (LOADS / 4), Q1_ = ((q) + 1) * (LOADS / 4);              \
        int p_ = (ks);                                                                     \
        if constexpr (ROTATE) {                                                            \
            p_ += rot;                                                                     \
            if (p_ >= nsteps) p_ -= nsteps;                                                \
        }                                                                                  \
        const int g_ = p_ / nk;                                                            \
        const int k0_ = (p_ - g_ * nk) * BK;                                               \
        const uint32_t sw_ = (uint32_t)((g_ * a.w_kseg + k0_) * 2u);                       \
        const uint32_t sx_ = (uint32_t)((g_ * a.x_kseg + k0_) * 2u);                       \
        const bool tail_ = ktail && k0_ + BK > K;                                          \
        CAAT_UNROLL for (int i = Q0_; i < Q1_; ++i) {                                      \
            const int c = cl ^ ((i * NW + wave) & 1);                                      \
            const uint32_t o = (!tail_ || k0_ + c * 8 < K) ? off[i] : OOB;                 \
            if (i < WLOADS) load_lds16_pol<WPOL>(rW, (Lb) + (i * NW + wave) * 64, o, sw_); \
            else load_lds16(rX, (Lb) + (i * NW + wave) * 64, o, sx_);                      \
        }                                                                                  \
        CAAT_SCHED_FENCE();                                                                \
    } while (0)

    f32x16 acc[IB][JB];
    // Fragment registers: two sets, sub-steps alternate between them, carried across K
    // steps (the end of a step reads the first fragments of the next).  The reads for
    // sub-step kk+1 are interleaved with the MFMAs of sub-step kk; each sub-step is a
    // scheduling region of its own, so the interleave slots can only take the next
    // sub-step's reads (otherwise the scheduler fills them with the current sub-step's
    // reads and waits on each one right before its MFMA).
    bf16x8 af[2][IB], bfr[2][JB];
#define CAAT_READ(q, Lb, kk)                                                               \
    do {                                                                                   \
        CAAT_UNROLL for (int i = 0; i < IB; ++i)                                           \
            af[q][i] = __builtin_bit_cast(bf16x8, (Lb)[aoff[kk] + i * 256]);               \
        CAAT_UNROLL for (int j = 0; j < JB; ++j)                                           \
            bfr[q][j] = __builtin_bit_cast(bf16x8, (Lb)[boff[kk] + j * 256]);              \
    } while (0)
#define CAAT_MMA(q, i0, i1)                                                                \
    do {                                                                                   \
        CAAT_UNROLL for (int i = (i0); i < (i1); ++i)                                      \
            CAAT_UNROLL for (int j = 0; j < JB; ++j)                                       \
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                       \
                    af[q][i], bfr[q][j], acc[i][j], 0, 0, 0);                              \
    } while (0)
    // nm MFMAs with NREAD fragment reads interleaved one to one, then a region fence.
#define CAAT_INTERLEAVE(nm)                                                                \
    do {                                                                                   \
        CAAT_UNROLL for (int r = 0; r < NREAD; ++r) {                                      \
            if (r < (nm)) CAAT_SCHED_GROUP(SG_MFMA, 1);                                    \
            CAAT_SCHED_GROUP(SG_DS_READ, 1);                                               \
        }                                                                                  \
        if ((nm) > NREAD) CAAT_SCHED_GROUP(SG_MFMA, (nm) - NREAD);                         \
        CAAT_SCHED_FENCE();                                                                \
    } while (0)
    // One K step on stage Lb whose sub-step 0 fragments are in set 0; Ln (the other
    // stage) receives step ks + 1.  The wait and the barrier follow the step's last
    // MFMAs, which gives step ks + 1 the whole step to land; the reads of its first
    // fragments follow the barrier (the SIMD's other wave covers them; placing the
    // barrier half way through the last sub-step, to hide them under this wave's own
    // MFMAs, measured 1-3 % slower with two waves per SIMD).  At the barrier every wave's
    // reads of Lb are complete, so the next step may refill Lb.
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
    // Four stages: step ks on Lb while steps ks + 1 and ks + 2 are in flight; Li (the stage
    // of step ks - 1, released by that step's barrier) receives step ks + 3.  The wait lets
    // only the two newest steps' loads (2 LOADS per lane) stay in flight, so step ks + 1
    // (in Ln) has landed at the barrier.  The four-stage tiles run one wave per SIMD, with
    // no second wave to compute while a wave waits to issue its loads, so step ks + 3's
    // loads go out a quarter at a time between the sub-steps' MFMAs (the 7B decode K1 at
    // T = 64: 46.7 -> 42.0 us, a four-stage shared-channel GEMM 29.4 -> 24.6 us; with two
    // waves per SIMD the same spread was 3-6 % slower, so the two-stage step keeps its
    // loads together).
    constexpr int VM_NEXT = 2 * LOADS;
    static_assert(NST == 2 || VM_NEXT < 64, "vmcnt range");
    // s_waitcnt encoding on gfx9: vmcnt[3:0] and vmcnt[5:4] at bits 15:14, expcnt (7: no
    // wait) at bits 6:4, lgkmcnt (0) at bits 11:8.
    constexpr int WAIT_NEXT = (VM_NEXT & 15) | ((VM_NEXT >> 4) << 14) | (7 << 4);
#define CAAT_STEP_MORE4(ks, Lb, Li, Ln)                                                    \
    do {                                                                                   \
        CAAT_ISSUE_Q(min((ks) + 3, nsteps - 1), Li, 0);                                    \
        CAAT_READ(1, Lb, 1); CAAT_MMA(0, 0, IB); CAAT_INTERLEAVE(NMFMA);                   \
        CAAT_ISSUE_Q(min((ks) + 3, nsteps - 1), Li, 1);                                    \
        CAAT_READ(0, Lb, 2); CAAT_MMA(1, 0, IB); CAAT_INTERLEAVE(NMFMA);                   \
        CAAT_ISSUE_Q(min((ks) + 3, nsteps - 1), Li, 2);                                    \
        CAAT_READ(1, Lb, 3); CAAT_MMA(0, 0, IB); CAAT_INTERLEAVE(NMFMA);                   \
        CAAT_ISSUE_Q(min((ks) + 3, nsteps - 1), Li, 3);                                    \
        CAAT_MMA(1, 0, IB);                                                                \
        CAAT_SCHED_FENCE();                                                                \
        __builtin_amdgcn_s_waitcnt(WAIT_NEXT);                                             \
        __builtin_amdgcn_s_barrier();                                                      \
        CAAT_SCHED_FENCE();                                                                \
        CAAT_READ(0, Ln, 0);                                                               \
    } while (0)
    // The last K step: no next step to load or read.
#define CAAT_STEP_LAST(Lb)                                                                 \
    do {                                                                                   \
        CAAT_READ(1, Lb, 1); CAAT_MMA(0, 0, IB); CAAT_INTERLEAVE(NMFMA);                   \
        CAAT_READ(0, Lb, 2); CAAT_MMA(1, 0, IB); CAAT_INTERLEAVE(NMFMA);                   \
        CAAT_READ(1, Lb, 3); CAAT_MMA(0, 0, IB); CAAT_INTERLEAVE(NMFMA);                   \
        CAAT_MMA(1, 0, IB);                                                                \
    } while (0)

    // Epilogue through LDS stage L1.  Accumulator element v of block (i, j) in lane l is
    // channel row 8 (v / 4) + 4 (l / 32) + v % 4 and token column l % 32 of that block.
    // Each wave writes its outputs (bf16, after the activation) into a [token][column]
    // image of the tile: 16-byte chunk C of image row r sits at C ^ (r & SWM), its 8-byte
    // halves swapped when bit 4 of r is set, which keeps both the 8-byte writes and the
    // 16-byte reads free of bank conflicts.  Then every thread stores whole 16-byte
    // chunks, and a wave's store covers whole token rows, instead of 8 bytes in each of
    // 32 rows.  An image larger than one stage goes through it in two passes of half the
    // tokens each.  Meanwhile L0 receives the next tile's first K step.
    constexpr int CPR = NCOL / 8;                    // 16-byte chunks per token row
    constexpr int SWM = (CPR < 16 ? CPR : 16) - 1;
    constexpr int NPASS = (BT * CPR + SLOTS - 1) / SLOTS;
    constexpr int PROWS = BT / NPASS;                // token rows per pass
    static_assert(NPASS <= 2 && PROWS * CPR <= SLOTS && PROWS % WT == 0 && WT % 32 == 0,
                  "the output image must fit one stage in at most two passes of whole waves");
    static_assert((PROWS * CPR) % NTH == 0, "output chunks must split evenly");
    constexpr int CPP = BN / 8;                      // pre-activation chunks per token row
    constexpr int SWP = (CPP < 16 ? CPP : 16) - 1;
    static_assert((BT / 2) * CPP <= SLOTS && (BT * CPP) % NTH == 0, "pre-activation image");

    int tile = xs + idx;
    int rot = ROTATE ? tile % nsteps : 0;
    int m, n0, t0;
    __amdgpu_buffer_rsrc_t rW, rX;
    uint32_t off[LOADS];
    CAAT_TILE_SETUP(tile, m, n0, t0, rW, rX, off);
    CAAT_ISSUE(0, L0);
    if constexpr (NST == 4) {
        CAAT_ISSUE(min(1, nsteps - 1), L1);
        CAAT_ISSUE(min(2, nsteps - 1), L2);
    }
    for (;;) {
        // The tile's first step has landed in L0; every wave has finished reading L1.
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __syncthreads();
        CAAT_UNROLL for (int i = 0; i < IB; ++i)
            CAAT_UNROLL for (int j = 0; j < JB; ++j)
                CAAT_UNROLL for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
        CAAT_READ(0, L0, 0);
        // Whole pairs of steps in the loop; an odd last step follows it.  With an even
        // count, the last step of the loop loads its own step again into the idle stage
        // (the load index is clamped), which nothing reads: one code path reaches the
        // epilogue from the loop and one from the last step, as few as the accumulators
        // can take without spilling.
        int kt = 0;
        if constexpr (NST == 4) {
            // Whole groups of four steps; the 1-3 remaining ones follow (step k is always
            // in stage k % 4, and a clamped load index refills a stage nothing reads).
            for (; kt + 4 <= nsteps; kt += 4) {
                CAAT_STEP_MORE4(kt, L0, L3, L1);
                CAAT_STEP_MORE4(kt + 1, L1, L0, L2);
                CAAT_STEP_MORE4(kt + 2, L2, L1, L3);
                CAAT_STEP_MORE4(kt + 3, L3, L2, L0);
            }
            const int rest = nsteps - kt;
            if (rest == 1) {
                CAAT_STEP_LAST(L0);
            } else if (rest == 2) {
                CAAT_STEP_MORE4(kt, L0, L3, L1);
                CAAT_STEP_LAST(L1);
            } else if (rest == 3) {
                CAAT_STEP_MORE4(kt, L0, L3, L1);
                CAAT_STEP_MORE4(kt + 1, L1, L0, L2);
                CAAT_STEP_LAST(L2);
            }
        } else {
            for (; kt + 2 <= nsteps; kt += 2) {
                CAAT_STEP_MORE(kt, L0, L1);
                CAAT_STEP_MORE(kt + 1, L1, L0);
            }
            if (kt < nsteps) CAAT_STEP_LAST(L0);
        }

        // The last step may have refilled a stage nothing reads; let it land and let
        // every wave finish its fragment reads.  Then the next tile's first step goes
        // to L0 while this tile's outputs pass through L1.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        // Lane-derived epilogue indices from an opaque copy of the thread index, so that
        // the compiler computes them here instead of holding them through the K loop.
        int te = tid;
        asm volatile("" : "+v"(te));
        const int r32e = te & 31, khe = (te >> 5) & 1;
        if (ACT && a.pre != nullptr) {
            // The raw pre-activation first, through an image over both stages (the first
            // half of the tokens in L0, the second in L1; all BN weight rows of the tile;
            // SwiGLU: the gate columns in image chunks [0, CPR), the up columns after).
            __bf16 *Pm = reinterpret_cast<__bf16 *>(a.pre) + (size_t)m * a.pre_stride;
            CAAT_UNROLL for (int j = 0; j < JB; ++j) {
                const int tb = wt * WT + j * 32;
                uint2 *img = reinterpret_cast<uint2 *>(tb < BT / 2 ? L0 : L1);
                const int r = tb % (BT / 2) + r32e;
                const int sw = r & SWP, hs = (r >> 4) & 1;
                CAAT_UNROLL for (int i = 0; i < IB; ++i) {
                    const int b32 = (wn * WN + i * 32) / 32;          // 32-row weight block
                    const int cb = (EPI == EPI_SWIGLU) ? (b32 & 1) * CPR + (b32 >> 1) * 4 : b32 * 4;
                    CAAT_UNROLL for (int g = 0; g < 4; ++g) {
                        bf16x4 o;
                        CAAT_UNROLL for (int q = 0; q < 4; ++q) o[q] = static_cast<__bf16>(acc[i][j][4 * g + q]);
                        img[(r * CPP + ((cb + g) ^ sw)) * 2 + (khe ^ hs)] = __builtin_bit_cast(uint2, o);
                    }
                }
            }
            __syncthreads();
            CAAT_UNROLL for (int it = 0; it < BT * CPP / NTH; ++it) {
                const int q = it * NTH + te;
                const int row = q / CPP, c = q % CPP;
                const int r = row % (BT / 2);
                uint4 v = (row < BT / 2 ? L0 : L1)[r * CPP + (c ^ (r & SWP))];
                if ((r >> 4) & 1) v = make_uint4(v.z, v.w, v.x, v.y);
                const int up = (EPI == EPI_SWIGLU) && c >= CPR;
                const int y = n0 + (c - up * CPR) * 8;
                const int t = t0 + row;
                if (t < T && y < N)
                    *reinterpret_cast<uint4 *>(Pm + (size_t)t * a.ld_pre + (up ? a.up_off : 0) + y) = v;
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __syncthreads();
        }

        // The next tile's first step into L0, under this tile's output image in L1.
        const int next = tile + nx;
        const bool more = next < xs + xc;
        int m2 = 0, n02 = 0, t02 = 0;
        __amdgpu_buffer_rsrc_t rW2 = rW, rX2 = rX;
        uint32_t off2[LOADS];
        if (more) {
            CAAT_TILE_SETUP(next, m2, n02, t02, rW2, rX2, off2);
            const int rot2 = ROTATE ? next % nsteps : 0;
            CAAT_ISSUE_T(0, L0, rW2, rX2, off2, rot2);
            if constexpr (NST == 4) {
                CAAT_ISSUE_T(min(1, nsteps - 1), L1, rW2, rX2, off2, rot2);
                CAAT_ISSUE_T(min(2, nsteps - 1), L2, rW2, rX2, off2, rot2);
            }
        }
        // The output image: the stage the next tile's first steps leave free.
        uint4 *const IMG = (NST == 4) ? L3 : L1;
        __bf16 *O = reinterpret_cast<__bf16 *>(a.out) + (size_t)m * a.o_stride;
        // EPI_RESID: every column goes to out2 with the addend; EPI_RESID_SPLIT: the columns
        // from a.split on, the others to out.
        constexpr bool RES = EPI == EPI_RESID || EPI == EPI_RESID_SPLIT;
        __bf16 *O2 = RES ? reinterpret_cast<__bf16 *>(a.out2) + (size_t)m * a.o_stride : O;
        constexpr int SITER = PROWS * CPR / NTH;         // 16-byte stores per thread and pass
        CAAT_UNROLL for (int ps = 0; ps < NPASS; ++ps) {
            // EPI_RESID: this pass's addend chunks, loaded where this thread stores, ahead
            // of the image so that their latency passes under it.
            uint4 rv[RES ? SITER : 1];
            if constexpr (RES) {
                const __bf16 *Rm = reinterpret_cast<const __bf16 *>(a.res) + (size_t)m * a.o_stride;
                CAAT_UNROLL for (int it = 0; it < SITER; ++it) {
                    const int q = it * NTH + te;
                    const int r = q / CPR, c = q % CPR;
                    const int t = t0 + ps * PROWS + r, n = n0 + c * 8;
                    rv[it] = (t < T && n < N && (EPI == EPI_RESID || n >= a.split))
                                 ? *reinterpret_cast<const uint4 *>(Rm + (size_t)t * a.ldo + n)
                                 : make_uint4(0u, 0u, 0u, 0u);
                }
            }
            CAAT_UNROLL for (int j = 0; j < JB; ++j) {
                const int tb = wt * WT + j * 32;                     // the 32 tokens' first row
                if (tb / PROWS != ps) continue;
                uint2 *img = reinterpret_cast<uint2 *>(IMG);
                const int r = tb % PROWS + r32e;                      // image row of the token
                const int sw = r & SWM, hs = (r >> 4) & 1;
                if (EPI == EPI_SWIGLU) {
                    CAAT_UNROLL for (int i = 0; i < IB; i += 2) {
                        const int cb = ((wn * IB + i) >> 1) * 4;      // first chunk of the 32 columns
                        CAAT_UNROLL for (int g = 0; g < 4; ++g) {
                            bf16x4 o;
                            CAAT_UNROLL for (int q = 0; q < 4; ++q)
                                o[q] = static_cast<__bf16>(silu(acc[i][j][4 * g + q]) * acc[i + 1][j][4 * g + q]);
                            img[(r * CPR + ((cb + g) ^ sw)) * 2 + (khe ^ hs)] = __builtin_bit_cast(uint2, o);
                        }
                    }
                } else {
                    CAAT_UNROLL for (int i = 0; i < IB; ++i) {
                        const int cb = (wn * WN + i * 32) / 8;
                        CAAT_UNROLL for (int g = 0; g < 4; ++g) {
                            bf16x4 o;
                            CAAT_UNROLL for (int q = 0; q < 4; ++q) {
                                float v = acc[i][j][4 * g + q];
                                if (EPI == EPI_GELU) v = gelu_erf(v);
                                if (EPI == EPI_GELU_TANH) v = gelu_tanh(v);
                                o[q] = static_cast<__bf16>(v);
                            }
                            img[(r * CPR + ((cb + g) ^ sw)) * 2 + (khe ^ hs)] = __builtin_bit_cast(uint2, o);
                        }
                    }
                }
            }
            __syncthreads();
            CAAT_UNROLL for (int it = 0; it < SITER; ++it) {
                const int q = it * NTH + te;
                const int r = q / CPR, c = q % CPR;
                uint4 v = IMG[r * CPR + (c ^ (r & SWM))];
                if ((r >> 4) & 1) v = make_uint4(v.z, v.w, v.x, v.y);
                const int t = t0 + ps * PROWS + r, n = n0 + c * 8;
                __bf16 *dst = O;
                if constexpr (RES) {
                    if (EPI == EPI_RESID || n >= a.split) {
                        const bf16x8 z = __builtin_bit_cast(bf16x8, v), rr = __builtin_bit_cast(bf16x8, rv[it]);
                        bf16x8 o;
                        CAAT_UNROLL for (int e = 0; e < 8; ++e)
                            o[e] = static_cast<__bf16>(fmaf(a.s_res, static_cast<float>(z[e]), static_cast<float>(rr[e])));
                        v = __builtin_bit_cast(uint4, o);
                        dst = O2;
                    }
                }
                if (t < T && n < N)
                    *reinterpret_cast<uint4 *>(dst + (size_t)t * a.ldo + n) = v;
            }
            if (ps + 1 < NPASS) {
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                __syncthreads();
            }
        }
        if (!more) break;
        tile = next; m = m2; n0 = n02; t0 = t02; rW = rW2; rX = rX2;
        rot = ROTATE ? tile % nsteps : 0;
        CAAT_UNROLL for (int i = 0; i < LOADS; ++i) off[i] = off2[i];
    }
#undef CAAT_READ
#undef CAAT_MMA
#undef CAAT_INTERLEAVE
#undef CAAT_STEP_MORE
#undef CAAT_STEP_LAST
#undef CAAT_STEP_MORE4
#undef CAAT_ISSUE
#undef CAAT_ISSUE_Q
#undef CAAT_ISSUE_T
#undef CAAT_TILE_SETUP
}

// Compute units of the current device (queried once).
int cu_count() {
    static const int n = [] {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 0;
        return cus > 0 ? cus : 256;
    }();
    return n;
}

// One launch of a kernel instance: at most as many workgroups as fit on the device at
// once (each then runs a sequence of tiles), and never more than the tiles.
template <int BN, int BT, int WGN, int WGT, int EPI, int NST>
hipError_t launch_epi(const GemmArgs &a, int tilesN, int tilesT, hipStream_t s) {
    constexpr int NTH = 64 * WGN * WGT;
    static const int resident = [] {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &n, reinterpret_cast<const void *>(&k_gemm_bf16<BN, BT, WGN, WGT, EPI, NST>), NTH,
                0) != hipSuccess || n < 1)
            n = 1;
        return n;
    }();
    const long total = (long)a.P * tilesN * tilesT;
    const long slots = (long)resident * cu_count();
    const dim3 grid((unsigned)(total < slots ? total : slots)), block(NTH);
    hipLaunchKernelGGL((k_gemm_bf16<BN, BT, WGN, WGT, EPI, NST>), grid, block, 0, s, a, tilesN, tilesT);
    return hipGetLastError();
}

template <int BN, int BT, int WGN, int WGT, int NST>
hipError_t launch(const GemmArgs &a, hipStream_t s) {
    const int ncol = (a.epi == EPI_SWIGLU) ? BN / 2 : BN;
    const int tilesN = (a.N + ncol - 1) / ncol;
    const int tilesT = (a.T + BT - 1) / BT;
    switch (a.epi) {
    case EPI_GELU: return launch_epi<BN, BT, WGN, WGT, EPI_GELU, NST>(a, tilesN, tilesT, s);
    case EPI_GELU_TANH: return launch_epi<BN, BT, WGN, WGT, EPI_GELU_TANH, NST>(a, tilesN, tilesT, s);
    case EPI_SWIGLU: return launch_epi<BN, BT, WGN, WGT, EPI_SWIGLU, NST>(a, tilesN, tilesT, s);
    // The residual epilogues serve prefill batches (T > 64) only, so the 64-token tiles
    // do not carry them; the per-rank one (EPI_RESID_SPLIT) runs only for P T h >= 2^25,
    // i.e. on thousands of 128 x 128 tiles, never on the four-stage form (<= 256 tiles).
    case EPI_RESID:
        if constexpr (BT == 64) return hipErrorInvalidValue;
        else return launch_epi<BN, BT, WGN, WGT, EPI_RESID, NST>(a, tilesN, tilesT, s);
    case EPI_RESID_SPLIT:
        if constexpr (BT == 64 || NST == 4) return hipErrorInvalidValue;
        else return launch_epi<BN, BT, WGN, WGT, EPI_RESID_SPLIT, NST>(a, tilesN, tilesT, s);
    default: return launch_epi<BN, BT, WGN, WGT, EPI_STORE, NST>(a, tilesN, tilesT, s);
    }
}

}  // namespace

bool gemm_bf16_rotates_k(const GemmArgs &a) { return a.T <= 64; }

bool gemm_bf16_supported(const GemmArgs &a) {
    // Byte offsets (over every K segment) are 32-bit and must stay below the OOB marker.
    const uint64_t wrows = (a.epi == EPI_SWIGLU) ? (uint64_t)a.up_off + a.N : (uint64_t)a.N;
    const uint64_t wspan = ((uint64_t)(a.kseg - 1) * a.w_kseg + wrows * a.K) * 2u;
    const uint64_t xspan = ((uint64_t)(a.kseg - 1) * a.x_kseg + (uint64_t)a.T * a.K) * 2u;
    return a.kseg >= 1 && wspan < OOB && xspan < OOB && a.K % 8 == 0 && a.N % 8 == 0 &&
           a.ldo % 8 == 0 && (a.kseg == 1 || a.epi == EPI_STORE);
}

// Tile choice: 256 x 256 with 8 waves (4 x 2, 64 x 128 each, two waves per SIMD so that
// one's fragment reads and waits are covered by the other's MFMAs) when there are at
// least two full waves of such tiles on the 256 CUs, or one full wave with a long
// contraction; else 128 x 128 with 4 waves so that smaller problems still spread over
// every CU.
//
// Where the big tiles would leave most of a last round empty, the small ones can finish
// first although they run at lower efficiency: with R rounds of big tiles (one per CU)
// against r rounds of small ones (two per CU, each a quarter of the work), the small
// tiles take r / 2 / E128 big-tile rounds, E128 = 0.77 being their measured efficiency
// relative to the big tiles (7B K1 shape: 939 against 1225 TFLOP/s).  They are chosen
// when that is less (a lone 7B K1 shard: 352 big tiles, 2 rounds, against
// 1408 small ones, 3 rounds: 177 against 186 us).
hipError_t gemm_bf16(const GemmArgs &a, hipStream_t s) {
    // Up to 64 tokens (the decode GEMMs the weight-streaming kernel leaves to this one):
    // 64-token tiles, so that no MFMA works on rows past the batch, with the stage rule of
    // the small tiles below.
    if (a.T <= 64) {
        const long ncol = (a.epi == EPI_SWIGLU) ? 64 : 128;
        const long tiles64 = (long)a.P * ((a.N + ncol - 1) / ncol);
        if (tiles64 <= cu_count()) return launch<128, 64, 2, 1, 4>(a, s);
        return launch<128, 64, 2, 1, 2>(a, s);
    }
    const int ncol256 = (a.epi == EPI_SWIGLU) ? 128 : 256;
    const int ncol128 = (a.epi == EPI_SWIGLU) ? 64 : 128;
    const long tiles256 = (long)a.P * ((a.N + ncol256 - 1) / ncol256) * ((a.T + 255) / 256);
    const long ktot = (long)a.K * a.kseg;
    if (tiles256 >= 512 || (tiles256 >= 256 && ktot >= 4096)) {
        const long tiles128 = (long)a.P * ((a.N + ncol128 - 1) / ncol128) * ((a.T + 127) / 128);
        const long cus = cu_count();
        const double big = (double)((tiles256 + cus - 1) / cus);
        const double small = (double)((tiles128 + 2 * cus - 1) / (2 * cus)) * 0.5 / 0.77;
        if (small >= big) return launch<256, 256, 4, 2, 2>(a, s);
    }
    // Small tiles.  Two workgroups per CU (two stages each) cover each other's load
    // latency; when there are no more tiles than CUs, each CU holds one workgroup anyway,
    // and four stages (three K steps in flight, 128 KB of LDS) cover it instead: the 1.1B
    // shared-channel GEMM at p = 0.25 (256 tiles, K = 8 x 704) 65.6 -> 52.0 us, the 130M one
    // (96 tiles) 35.2 -> 28.1 us; with more tiles than CUs the four-stage form was slower
    // everywhere (130M K1, 768 tiles: 34.8 against 43.4 us).
    const long ncol = (a.epi == EPI_SWIGLU) ? 64 : 128;
    const long tiles128 = (long)a.P * ((a.N + ncol - 1) / ncol) * ((a.T + 127) / 128);
    if (tiles128 <= cu_count()) return launch<128, 128, 2, 2, 4>(a, s);
    return launch<128, 128, 2, 2, 2>(a, s);
}

}  // namespace caat
