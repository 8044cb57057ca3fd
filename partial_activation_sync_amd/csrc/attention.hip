// Attention core of the full block: causal softmax attention of every head of every
// rank, bf16 in and out, fp32 scores and accumulation.
//
// "Tensor-Parallelism with Partially Synchronized Activations", App. A.1 Eq. 16 / 18 and
// App. A.2 Eq. 24: rank m computes its heads' outputs H_m = Attention(X_m W^Q_m,
// X_m W^K_m, X_m W^V_m) from its own input X_m; with partially synchronized
// activations the inputs differ per rank, and all ranks run on this device (§3.2).
//
// One workgroup (4 waves) takes 128 queries of one head of one rank, and two workgroups
// share a CU (two waves per SIMD, 80 KB of LDS each); each wave holds 32 queries' Q
// fragments in registers for the whole key loop.  Keys come in blocks of 64 through two
// LDS stages (K tile [64 keys][d] and V^T tile [d][64 keys], both filled by buffer loads
// that write LDS directly, rows padded by one 16-byte slot).
// Per block and wave:
//   S^T = K Q^T     (v_mfma_f32_32x32x16_bf16, keys as rows, queries as columns), so
//                   each lane's accumulators hold one query's scores for 16 keys and the
//                   row statistics of the online softmax need only the lane pair l, l^32;
//                   MFMA row rho computes key rho with bits 2 and 3 exchanged, so that
//                   accumulator element v of lane l holds key 16 (v / 8) + 8 g + v % 8
//                   (g = l / 32) of its 32-key block;
//   mask keys past the query or past the sequence (only on the wave's diagonal block),
//   update the running max in log2 units (scale log2(e)/sqrt(d) folded into the exp2
//   argument), and rescale the output only when some query's max grew by more than 8
//   (a stale max leaves every probability at most 2^8, which fp32 sums and bf16 holds);
//   O^T += V^T P^T  with P^T taken straight from the S^T accumulators (bf16) as the
//                   column operand: lane l's 8 values of a 16-key chunk are its keys
//                   8g..8g+7, so each V^T fragment is one 16-byte LDS read of 8
//                   consecutive keys.
// A wave skips key blocks that lie wholly past its last query; the workgroup's loads and
// barriers run for all of them.  The two workgroups of a CU synchronize independently, so
// one's softmax arithmetic overlaps the other's matrix products.  Queries past the
// sequence and keys past it read as zero
// (buffer range checks) and are masked; sequences never see each other.
#include "caat_internal.h"
#include "bufload.h"

#if defined(__HIP_DEVICE_COMPILE__)
#define CAAT_UNROLL _Pragma("unroll")
#else
#define CAAT_UNROLL
#endif

namespace caat {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int NW = 4, NT = 64 * NW, BQ = 32 * NW, BKV = 64;

template <int D>
__global__ __launch_bounds__(NT, 2)
void k_attn(AttnArgs a, int nqb, int ngrp)
{
    constexpr int CK = D / 8;                 // 16-byte chunks per K row
    constexpr int KROW = CK + 1;              // K row pitch in slots (one slot of padding)
    constexpr int VROW = BKV / 8 + 1;         // V^T row pitch in slots (8 chunks + padding)
    constexpr int KLOADS = (BKV * KROW + NT - 1) / NT, VLOADS = (D * VROW + NT - 1) / NT;
    constexpr int KSLOTS = KLOADS * NT, VSLOTS = VLOADS * NT;
    constexpr int NKK = D / 16;               // MFMA steps over d for the scores
    constexpr int NDB = D / 32;               // 32-row blocks of O^T
    __shared__ __attribute__((aligned(16))) uint4 K0[KSLOTS];
    __shared__ __attribute__((aligned(16))) uint4 K1[KSLOTS];
    __shared__ __attribute__((aligned(16))) uint4 V0[VSLOTS];
    __shared__ __attribute__((aligned(16))) uint4 V1[VSLOTS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Dispatch order: every (rank, head, sequence) group's longest query block first, then
    // the next longest.  Consecutive workgroups go to the 8 XCDs in turn, so with a
    // multiple of 8 groups each XCD keeps to the same groups and its L2 serves their keys.
    const int grp = blockIdx.x % ngrp;
    const int qb = nqb - 1 - (int)(blockIdx.x / ngrp);
    const int nseq = a.T / a.S;
    const int sq = grp % nseq, hd = (grp / nseq) % a.nh, m = grp / (nseq * a.nh);
    const int T = a.T, S = a.S, nh = a.nh, Tp = a.Tp;
    const int ld = 3 * nh * D;
    const int seq0 = sq * S, ql0 = qb * BQ;

    const __bf16 *QKV = reinterpret_cast<const __bf16 *>(a.qkv) + (size_t)m * T * ld;
    const __amdgpu_buffer_rsrc_t rQ = make_rsrc(QKV, (uint32_t)((size_t)T * ld * 2u));
    const __bf16 *VT = reinterpret_cast<const __bf16 *>(a.vt) + ((size_t)m * nh + hd) * D * Tp;
    const __amdgpu_buffer_rsrc_t rV = make_rsrc(VT, (uint32_t)((size_t)D * Tp * 2u));

    // Q fragments (column operand of S^T): query ql, d values 16 kk + 8 (lane / 32) ...
    const int wq0 = ql0 + wave * 32;          // the wave's first query
    const int ql = wq0 + (lane & 31);
    const int g = lane >> 5;
    bf16x8 qf[NKK];
    {
        const uint32_t qoff = (uint32_t)(((size_t)(seq0 + ql) * ld + (size_t)hd * D + 8 * g) * 2u);
        CAAT_UNROLL for (int kk = 0; kk < NKK; ++kk)
            qf[kk] = load16(rQ, ql < S ? qoff + kk * 32u : OOB);
    }
    // Last key the wave needs (-1: every query of the wave lies past the sequence).
    const int wlast = wq0 < S ? min(wq0 + 31, S - 1) : -1;

    // Tile loads: load i of a wave writes the 64 slots from (i * NT + 64 wave) on, lane
    // by lane, so slot s = i * NT + tid holds chunk s % pitch of row s / pitch.  Rows
    // are padded by one slot (loaded out of range, as zero) so that the fragment reads
    // of 16 consecutive rows fall in distinct banks while every read of a row is one base
    // address plus an immediate offset.  The K descriptor of a block starts at its first
    // key and ends with the sequence, so rows past the sequence read as zero with no
    // per-lane test; V^T rows are tested per 8-key chunk against the keys left.
    uint32_t koff[KLOADS];
    CAAT_UNROLL for (int i = 0; i < KLOADS; ++i) {
        const int s = i * NT + tid, r = s / KROW, c = s % KROW;
        koff[i] = (r < BKV && c < CK) ? (uint32_t)((r * ld + c * 8) * 2) : OOB;
    }
    uint32_t voff[VLOADS];
    int vkey[VLOADS];
    CAAT_UNROLL for (int i = 0; i < VLOADS; ++i) {
        const int s = i * NT + tid, dr = s / VROW, c = s % VROW;
        const bool in = dr < D && c < BKV / 8;
        vkey[i] = in ? c * 8 : BKV;            // padding: never below the keys left
        voff[i] = in ? (uint32_t)((dr * Tp + c * 8) * 2) : OOB;
    }
    const __bf16 *Kseq = QKV + (size_t)seq0 * ld + (size_t)(nh + hd) * D;
#define CAAT_ISSUE(kv0, Kb, Vb)                                                            \
    do {                                                                                   \
        const int left_ = S - (kv0);                                                       \
        const __amdgpu_buffer_rsrc_t rK_ = make_rsrc(                                      \
            Kseq + (size_t)(kv0) * ld, left_ > 0 ? (uint32_t)left_ * (uint32_t)ld * 2u : 0u); \
        CAAT_UNROLL for (int i = 0; i < KLOADS; ++i)                                       \
            load_lds16(rK_, (Kb) + i * NT + wave * 64, koff[i], 0);                        \
        CAAT_UNROLL for (int i = 0; i < VLOADS; ++i)                                       \
            load_lds16(rV, (Vb) + i * NT + wave * 64, vkey[i] < left_ ? voff[i] : OOB,     \
                       (uint32_t)(seq0 + (kv0)) * 2u);                                     \
    } while (0)

    f32x16 acc_o[NDB];
    CAAT_UNROLL for (int b = 0; b < NDB; ++b)
        CAAT_UNROLL for (int v = 0; v < 16; ++v) acc_o[b][v] = 0.f;
    // Running max in log2 units (score * sc) and running sum of 2^(score * sc - m_run).
    float m_run = -INFINITY, l_run = 0.f;
    const float sc = 1.44269504088896341f / sqrtf((float)D);
    // K tile row of the lane's S^T MFMA row: bits 2 and 3 of the row exchanged.
    const int krho = ((lane & 31) & ~12) | ((lane & 4) << 1) | ((lane & 8) >> 1);
    constexpr float RESCALE_MARGIN = 8.f;

    // One key block on the stage (Kb, Vb).  MASK: the block holds keys past one of the
    // wave's queries or past the sequence (the wave's diagonal block).
#define CAAT_BLOCK(kv0, Kb, Vb, MASK)                                                      \
    do {                                                                                   \
        f32x16 acc_s[2];                                                                   \
        CAAT_UNROLL for (int kb = 0; kb < 2; ++kb) {                                       \
            CAAT_UNROLL for (int v = 0; v < 16; ++v) acc_s[kb][v] = 0.f;                   \
            const uint4 *krow_ = (Kb) + (kb * 32 + krho) * KROW + g;                       \
            CAAT_UNROLL for (int kk = 0; kk < NKK; ++kk) {                                 \
                const bf16x8 kf = __builtin_bit_cast(bf16x8, krow_[2 * kk]);               \
                acc_s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], acc_s[kb], \
                                                                    0, 0, 0);              \
            }                                                                              \
        }                                                                                  \
        float mb = -INFINITY;                                                              \
        CAAT_UNROLL for (int kb = 0; kb < 2; ++kb)                                         \
            CAAT_UNROLL for (int v = 0; v < 16; ++v) {                                     \
                if (MASK) {                                                                \
                    const int key = (kv0) + kb * 32 + 16 * (v >> 3) + 8 * g + (v & 7);     \
                    if (key > ql || key >= S) acc_s[kb][v] = -INFINITY;                    \
                }                                                                          \
                mb = fmaxf(mb, acc_s[kb][v]);                                              \
            }                                                                              \
        mb = fmaxf(mb, __shfl_xor(mb, 32, 64)) * sc;                                       \
        const bool grow = mb > m_run + RESCALE_MARGIN;                                     \
        const float m_new = grow ? mb : m_run;                                             \
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);                         \
        float ls = 0.f;                                                                    \
        bf16x8 pf[4];                                                                      \
        CAAT_UNROLL for (int kb = 0; kb < 2; ++kb)                                         \
            CAAT_UNROLL for (int v = 0; v < 16; ++v) {                                     \
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(acc_s[kb][v], sc, -m_new)); \
                ls += p;                                                                   \
                pf[kb * 2 + (v >> 3)][v & 7] = static_cast<__bf16>(p);                     \
            }                                                                              \
        ls += __shfl_xor(ls, 32, 64);                                                      \
        l_run = alpha * l_run + ls;                                                        \
        m_run = m_new;                                                                     \
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {                                      \
            CAAT_UNROLL for (int b = 0; b < NDB; ++b)                                      \
                CAAT_UNROLL for (int v = 0; v < 16; ++v) acc_o[b][v] *= alpha;             \
        }                                                                                  \
        CAAT_UNROLL for (int b = 0; b < NDB; ++b) {                                        \
            const uint4 *vrow = (Vb) + (b * 32 + (lane & 31)) * VROW + g;                  \
            CAAT_UNROLL for (int kc = 0; kc < 4; ++kc) {                                   \
                const bf16x8 vf = __builtin_bit_cast(bf16x8, vrow[2 * kc]);                \
                acc_o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kc], acc_o[b],   \
                                                                   0, 0, 0);               \
            }                                                                              \
        }                                                                                  \
    } while (0)

    const int kv_end = min(S, ql0 + BQ);
    const int nkv = (kv_end + BKV - 1) / BKV;
    // Blocks wholly before the workgroup's first query (and inside the sequence) need no
    // mask for any wave; they run in a loop without branches, so the output accumulators
    // stay in place.  The last blocks (at most two, plus one for a ragged sequence) run
    // masked, and a wave skips those that lie wholly past its last query.
    const int nfull = min(ql0, S) / BKV;
    // Two stages: block j + 1's loads are issued at the start of block j, and the
    // barrier after the wait both publishes them and frees the stage block j read.
#define CAAT_NEXT()                                                                        \
    do {                                                                                   \
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");                                   \
        __syncthreads();                                                                   \
    } while (0)
    CAAT_ISSUE(0, K0, V0);
    CAAT_NEXT();
    int j = 0;
    for (; j + 2 <= nfull; j += 2) {
        CAAT_ISSUE((j + 1) * BKV, K1, V1);
        CAAT_BLOCK(j * BKV, K0, V0, false);
        CAAT_NEXT();
        CAAT_ISSUE((j + 2) * BKV, K0, V0);
        CAAT_BLOCK((j + 1) * BKV, K1, V1, false);
        CAAT_NEXT();
    }
    for (; j < nkv; j += 2) {
        CAAT_ISSUE((j + 1) * BKV, K1, V1);
        if (j * BKV <= wlast) CAAT_BLOCK(j * BKV, K0, V0, true);
        CAAT_NEXT();
        CAAT_ISSUE((j + 2) * BKV, K0, V0);
        if ((j + 1) * BKV <= wlast) CAAT_BLOCK((j + 1) * BKV, K1, V1, true);
        CAAT_NEXT();
    }
#undef CAAT_NEXT
#undef CAAT_ISSUE
#undef CAAT_BLOCK

    if (ql >= S) return;
    const float inv = 1.0f / l_run;
    __bf16 *Hrow = reinterpret_cast<__bf16 *>(a.H) + ((size_t)m * T + seq0 + ql) * nh * D +
                   (size_t)hd * D;
    // Accumulator element v of block b in lane l is d = 32 b + 8 (v / 4) + 4 (l / 32) + v % 4.
    CAAT_UNROLL for (int b = 0; b < NDB; ++b)
        CAAT_UNROLL for (int q4 = 0; q4 < 4; ++q4) {
            bf16x4 o;
            CAAT_UNROLL for (int e = 0; e < 4; ++e) o[e] = static_cast<__bf16>(acc_o[b][4 * q4 + e] * inv);
            *reinterpret_cast<bf16x4 *>(Hrow + b * 32 + 8 * q4 + 4 * g) = o;
        }
}

}  // namespace

hipError_t attention_bf16(const AttnArgs &a, hipStream_t s) {
    const int nqb = (a.S + BQ - 1) / BQ;
    const int ngrp = (a.T / a.S) * a.nh * a.P;
    const dim3 grid(nqb * ngrp), block(NT);
    if (a.d == 128)
        hipLaunchKernelGGL(k_attn<128>, grid, block, 0, s, a, nqb, ngrp);
    else
        hipLaunchKernelGGL(k_attn<64>, grid, block, 0, s, a, nqb, ngrp);
    return hipGetLastError();
}

}  // namespace caat
