// Internal declarations shared by the libcaat sources (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "caat.h"

struct caat_ctx {
    int h;        // hidden size
    int ffn;      // full FFN size (0 for the out-projection)
    int P;        // emulated tensor-parallel ranks
    int fs;       // ffn / P: Y columns per rank
    int F1;       // W1 rows per rank: fs, or 2 fs for SwiGLU
    int kin;      // input width: h (MLP) or h / P (out-projection)
    int k2;       // contraction length of the row-parallel GEMM: fs or h / P
    int n_s;      // shared channels [0, n_s)
    int norm;     // caat_norm
    int act;      // caat_act
    int dtype;    // caat_dtype
    double p;     // sync fraction as given
    float eps;    // normalization epsilon
    float s_priv; // private channel scale
    void *ws;     // caller's workspace
    size_t ws_bytes;
};

namespace caat {

// Epilogues of the GEMM kernels.
// EPI_RESID: out2 = res + s_res * bf16(acc) (one fused multiply-add) for every column;
// EPI_RESID_SPLIT: the same for columns n >= split, out = bf16(acc) for the others.  res
// and out2 are laid out like out (bf16 MFMA kernel only).
enum Epilogue { EPI_STORE = 0, EPI_GELU = 1, EPI_GELU_TANH = 2, EPI_SWIGLU = 3, EPI_RESID = 4,
                EPI_RESID_SPLIT = 5 };

// One batched "NT" GEMM: for every batch index m < P, token t < T and column n < N,
//   acc = sum_{g < kseg} sum_{k < K} W[m][g][row(n)][k] * X[m][g][t][k]
// and out[m][t][n] = epilogue(acc).  kseg > 1 concatenates K segments (the emulated
// ranks' contractions, summed in the accumulator).  For EPI_SWIGLU, N counts Y columns
// and column n uses W rows n (gate) and up_off + n (up): out = silu(gate) * up.
struct GemmArgs {
    int P, N, T, K;
    const void *W;  size_t w_stride;   // elements between batches; rows of K elements
    const void *X;  size_t x_stride;   // elements between batches; rows of K elements
    void *out;      size_t o_stride;   // elements between batches
    int ldo;                           // elements between output rows (tokens)
    int up_off;                        // SwiGLU: W row offset of the up projection
    int epi;
    int kseg;                          // K segments (>= 1)
    size_t w_kseg, x_kseg;             // elements between K segments
    // Optional second output of an activation epilogue (nullptr: none): the raw
    // pre-activation, [t][F1] per batch with row stride ld_pre (SwiGLU: gate columns
    // [0, N), up columns [up_off, up_off + N)).  Only the bf16 MFMA kernel writes it.
    void *pre;      size_t pre_stride;
    int ld_pre;
    // EPI_RESID(_SPLIT): the first column (a multiple of 8) that takes the addend (split
    // only), the addend and that part's output (same batch stride and row stride as out),
    // and the factor of the accumulator (rounded to bf16 first).
    int split;
    const void *res;
    void *out2;
    float s_res;
};

hipError_t gemm_bf16(const GemmArgs &a, hipStream_t s);

// out[b][m][n] = sum_k A[b][k][m] B[b][k][n], bf16 in and out, fp32 accumulation: the
// contraction runs across rows of two token-major operands (row strides lda, ldb,
// elements; batch strides in elements).  M, N, lda, ldb, ldo multiples of 8.
struct TnArgs {
    int P, M, N, K;
    const void *A;  size_t a_stride;  int lda;
    const void *B;  size_t b_stride;  int ldb;
    void *out;      size_t o_stride;  int ldo;
};
bool gemm_tn_supported(const TnArgs &a);
hipError_t gemm_tn_bf16(const TnArgs &a, hipStream_t s);
hipError_t gemm_f32(const GemmArgs &a, hipStream_t s);
bool gemm_bf16_supported(const GemmArgs &a);
// Whether the bf16 MFMA kernel walks each tile's K steps in a per-tile rotated order for
// this GEMM (its 64-token tiles do): its sums then round differently from the same
// contraction tiled another way, e.g. a pre-activation stored by the activation
// epilogue against the backward's recompute as a plain GEMM.
bool gemm_bf16_rotates_k(const GemmArgs &a);
// Weight-streaming variant for decode batches, bf16: the GEMMs of up to 64 tokens for
// which gemm_decode_applies (the others take the MFMA kernel's 64-token tiles).
bool gemm_decode_applies(const GemmArgs &a);
hipError_t gemm_decode_bf16(const GemmArgs &a, hipStream_t s);

// S (nullable): the shared channels already reduced over ranks, [T][s_ld] with
// s_ld >= n_s; when S is set only the private columns of the partials are read.
struct PsyncArgs {
    int P, T, h, n_s, norm;
    float s_priv, eps;
    const void *partials, *resid, *gamma, *beta;
    void *out, *out_resid;
    const void *S;
    int s_ld;
    // When non-null, the residual rows r of the private channel chunks (from n_s rounded
    // up to 8; with S, n_s % 8 == 0) are already final there (the row GEMM's epilogue
    // added the residual; it is out_resid), so K3 reads them instead of the partials and
    // the residual, and does not write them.  Only where psync_reads_final_private holds.
    const void *priv_r;
};

hipError_t psync_norm(const PsyncArgs &a, int dtype, hipStream_t s);
// Whether psync_norm accepts priv_r for P ranks and rows of h channels (bf16, where the
// single-pass kernel runs; the multi-pass kernel for wider rows does not take them).
bool psync_reads_final_private(int P, int h, int dtype);

}  // namespace caat

// ---------------------------------------------------------------------------------
// Backward of the sublayer.
namespace caat {

// B3: the norm derivative of every rank, then the reduce over ranks of the shared
// channels of the result (the placement after the norm derivative), per token; the
// norm parameters' gradients are accumulated per workgroup into gpart / bpart
// [nblk][h] (fp32) and summed by colsum_f32.
struct PsyncBwdArgs {
    int P, T, h, n_s, norm;
    float s_priv, eps;
    const void *r;       // [P][T][h] forward out_resid (r = R + Z)
    const void *dout;    // [P][T][h]
    const void *dres;    // [P][T][h] or NULL (zero)
    const void *gamma;   // [h]
    void *dzt;           // [P][T][h] gradient of the partials
    void *dresid;        // [P][T][h] or NULL
    float *gpart, *bpart;
    int nblk;
};
int psync_bwd_blocks(int T);
hipError_t psync_norm_bwd(const PsyncBwdArgs &a, int dtype, hipStream_t s);
// out[l] = sum over r < rows (ascending) of part[r][l], fp32.
hipError_t colsum_f32(const float *part, int rows, int h, float *out, hipStream_t s);
// dst[b][c][r] = src[b][r][c] for r < R, 0 for R <= r < Rp (Rp % 8 == 0, Rp >= R).
hipError_t transpose(const void *src, void *dst, int B, int R, int C, int Rp, int dtype,
                     hipStream_t s);
// The same for source rows `pitch` elements apart and batches `bstride` elements apart
// (pitch % 8 == 0): dst[b][c][r] = src[b * bstride + r * pitch + c].
hipError_t transpose_strided(const void *src, void *dst, int B, int R, int C, int Rp, int pitch,
                             size_t bstride, int dtype, hipStream_t s);
// Activation backward over rows of the pre-activation A [rows][F1]:
//   da = dY * sigma'(A) ([rows][F1]; SwiGLU: gate and up halves), Y = sigma(A)
//   ([rows][fs]).
hipError_t act_backward(int act, int dtype, size_t rows, int fs, const void *A, const void *dY,
                        void *da, void *Y, hipStream_t s);
// dst[i] += src[i], n % 8 == 0.
hipError_t add_inplace(void *dst, const void *src, size_t n, int dtype, hipStream_t s);

}  // namespace caat

// ---------------------------------------------------------------------------------
// Attention core of the full block (bf16): causal softmax attention per head.
namespace caat {
struct AttnArgs {
    int P, T, S, nh, d;     // ranks, tokens, sequence length (T % S == 0), heads per rank, width
    const void *qkv;        // [P][T][3 nh d]: Q, K, V of the rank's heads
    const void *vt;         // [P][nh][d][Tp]: V transposed, Tp = T rounded up to 8
    int Tp;
    void *H;                // [P][T][nh d]
};
hipError_t attention_bf16(const AttnArgs &a, hipStream_t s);
}  // namespace caat
