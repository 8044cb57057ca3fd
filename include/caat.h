/*
 * caat.h - C ABI of libcaat: the forward pass of one CAAT tensor-parallel sublayer
 * (partially synchronized activations) on an AMD Instinct MI355X (gfx950), with all
 * P tensor-parallel ranks emulated on the one device.
 *
 * Method: "Tensor-Parallelism with Partially Synchronized Activations"
 * (Lamprecht, Karnieli, Hanani, Giladi, Soudry).
 *   - MLP sublayer: App. A.2, Eq. 22 (P = 2: §3.1, Eq. 6-8).  Rank m computes
 *       Zt_m = act(X_m A_m) B_m       (column-parallel A, row-parallel B)
 *   - Attention output projection: App. A.2, Eq. 24 (P = 2: App. A.1, Eq. 19).
 *       Zt_m = H_m O_m                (O row-parallel; rank m holds all h columns)
 *   - Partial channel-reduce (Eq. 22 / 24): for channel l < n_s = floor(h p),
 *       Z_m[l] = sum over ranks of Zt[l]; otherwise Z_m[l] = s_priv * Zt_m[l].
 *     The shared channels are the first n_s (§3).  s_priv is the private channel
 *     scaling of §4 (Eq. 14-15); it is 1 unless set.
 *   - Then, per rank, the residual add and the normalization (§4, Eq. 9):
 *       r_m = R_m + Z_m,  out_m = Norm(r_m)
 *     LayerNorm: (r - mean) / sqrt(var + eps) * gamma + beta (biased variance).
 *     RMSNorm:   r / sqrt(mean(r^2) + eps) * gamma.
 *   - All ranks run on one device, one after another in the page's terms
 *     ("logical devices", §3.2), so the channel-reduce is a local sum.
 *
 * Conventions for every call below.
 *   Pointers: device pointers (HBM) unless stated; 16-byte aligned; dense,
 *     row-major, in the handle's dtype (CAAT_BF16: bfloat16, CAAT_F32: float).
 *     The caller owns every buffer; the library never allocates device memory.
 *   Shapes (h hidden size, P ranks, T tokens, f_s = ffn / P):
 *     x / in     [P][T][h]       (act = CAAT_NONE: the head outputs H, [P][T][h/P])
 *     W1         [P][F1][h]      F1 = f_s, or 2 f_s for SwiGLU: rows [0, f_s) are the
 *                                gate and rows [f_s, 2 f_s) the up projection of the
 *                                same column range of the full matrices.  Row k of
 *                                shard m is column k of A_m.  Unused for CAAT_NONE.
 *     W2         [P][h][k2]      k2 = f_s (MLP) or h/P (out-projection).  Row l of
 *                                shard m is column l of B_m (or of O_m).
 *     Y          [P][T][f_s]     activation after the first GEMM (workspace)
 *     partials   [P][T][h]       Zt before any reduction (workspace)
 *     resid, out, out_resid  [P][T][h]
 *     gamma, beta [h]            shared by all ranks; beta is used by LayerNorm only
 *   Streams: `stream` is a hipStream_t (NULL = the default stream).  Every call
 *     only enqueues kernels on it and returns without a host synchronisation.
 *   Errors: every call returns a caat_status.  Arguments are checked before any
 *     launch; a call that returns an error has enqueued nothing.  A failed launch
 *     returns CAAT_EDEVICE.  Faults during execution surface at the caller's next
 *     synchronisation of the stream.  No C++ exception crosses this interface.
 *     Two environment variables, read on the host by every call that would launch
 *     (after its argument checks, before any HIP call), force the device error paths
 *     for tests: CAAT_FAULT=launch makes the call return CAAT_EDEVICE, as a failed
 *     launch does, with nothing enqueued; CAAT_ARCH=<gfx name> other than gfx950
 *     makes it return CAAT_EUNSUPPORTED, as on another architecture.
 *   Concurrency: calls on one handle that overlap on different streams must use
 *     different workspaces (one handle per stream).
 *   Aliasing: in the forward calls, out_resid or out may be the resid buffer itself
 *     (the residual stream updated in place; each element is read before it is written,
 *     by the same thread); no other output may overlap an input or another output.
 */
#ifndef CAAT_H
#define CAAT_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct caat_ctx *caat_handle;

typedef enum {
    CAAT_OK = 0,
    CAAT_EINVAL = -1,       /* bad argument: null pointer, bad shape, misalignment */
    CAAT_ENOMEM = -2,       /* host allocation of the handle failed */
    CAAT_EWORKSPACE = -3,   /* no workspace set, or smaller than caat_workspace_bytes */
    CAAT_EDEVICE = -4,      /* a HIP call or kernel launch failed */
    CAAT_EUNSUPPORTED = -5  /* not a gfx950 device, or a size beyond the kernels' limits */
} caat_status;

typedef enum { CAAT_LAYERNORM = 0, CAAT_RMSNORM = 1 } caat_norm;

/* sigma of Eq. 20-22.  CAAT_GELU: a * Phi(a) (erf form).  CAAT_GELU_TANH: the tanh
 * approximation of GeLU.  CAAT_SWIGLU: silu(x A_gate) * (x A_up).  CAAT_NONE: the
 * attention output projection (no first GEMM, no activation). */
typedef enum { CAAT_GELU = 0, CAAT_GELU_TANH = 1, CAAT_SWIGLU = 2, CAAT_NONE = 3 } caat_act;

typedef enum { CAAT_F32 = 0, CAAT_BF16 = 1 } caat_dtype;

/* Creates a handle for one sublayer shape.  Host only: touches no device.
 *   h: hidden size, 8 <= h <= 16384, h % 8 == 0.
 *   ffn: FFN size of the full MLP, ffn % P == 0, (ffn / P) % 8 == 0; ignored for
 *        CAAT_NONE, which instead needs (h / P) % 8 == 0.
 *   P: emulated ranks, 1..16.  p: sync fraction in [0, 1] (NaN rejected).
 *   n_s = floor(h p) shared channels (an h p within 1e-9 h of an integer counts as
 *   that integer), see caat_shared_channels.
 * Returns CAAT_EINVAL on a bad argument, CAAT_ENOMEM if the handle cannot be made. */
int caat_create(caat_handle *out, int h, int ffn, int P, double p, int norm, int act,
                int dtype);

/* Frees the handle (not the caller's buffers).  NULL is accepted. */
int caat_destroy(caat_handle handle);

/* Normalization epsilon (default 1e-5), eps >= 0. */
int caat_set_eps(caat_handle handle, float eps);

/* Private channel scale s_priv (default 1; the page's setting is sqrt(P), §4). */
int caat_set_private_scale(caat_handle handle, float s);

/* n_s, the number of shared channels [0, n_s); or CAAT_EINVAL for a NULL handle. */
int caat_shared_channels(caat_handle handle);

/* Bytes of device workspace a forward over T tokens needs: Y, the partials and (when
 * n_s % 8 == 0) the reduced shared channels S.  Returns 0 for a NULL handle or T < 1. */
size_t caat_workspace_bytes(caat_handle handle, int T);

/* Attaches caller-owned device memory as the workspace (16-byte aligned). */
int caat_set_workspace(caat_handle handle, void *dev_ptr, size_t bytes);

/* Whole sublayer, residual = the input x (MLP only; Eq. 9 with R = X):
 * x [P][T][h] -> out [P][T][h].  Needs a workspace of caat_workspace_bytes(T). */
int caat_forward(caat_handle handle, int T, const void *x, const void *W1, const void *W2,
                 const void *gamma, void *out, void *stream);

typedef struct {
    int T;
    const void *in;      /* x [P][T][h], or H [P][T][h/P] for CAAT_NONE */
    const void *resid;   /* R [P][T][h]; NULL means resid = in (MLP only) */
    const void *W1;      /* NULL for CAAT_NONE */
    const void *W2;
    const void *gamma;
    const void *beta;    /* NULL means zero (LayerNorm) */
    void *out;           /* Norm(r) [P][T][h] */
    void *out_resid;     /* r = R + Z [P][T][h], the next residual; NULL: not stored */
    void *stream;
} caat_args;

/* Whole sublayer with an explicit residual, beta and residual output.  The attention
 * out-projection (CAAT_NONE) must come through here, since its input is not [P][T][h]. */
int caat_forward_ex(caat_handle handle, const caat_args *args);

/* The steps of a sublayer forward, in launch order (for caat_forward_timed's events):
 *   0 column-parallel GEMM + activation (nothing for CAAT_NONE)
 *   1 row-parallel GEMM: every rank's partials, or, on the fused path (see
 *     caat_row_gemm_reduce and caat_forward_fused), the GEMM whose accumulators sum the
 *     shared channels over the ranks
 *   2 fused path: the GEMM of the private channels (nothing otherwise)
 *   3 partial channel-reduce (or S on the fused path), private scaling, residual, norm */
#define CAAT_FWD_STEPS 4

/* Size of the library's static device workspace (caat_forward_scratch): 64 MiB per
 * device, enough for caat_workspace_bytes(T) of a 7B decode batch (T <= 64: under 6 MB)
 * or a 130M-sized prefill of 4096 tokens (54 MB). */
#define CAAT_SCRATCH_BYTES (64u << 20)

/* caat_forward_ex for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels and
 * results, with the workspace taken from a static array inside the library instead of
 * the handle's caat_set_workspace memory.  Allocates nothing, and calls nothing that
 * allocates.  The array is CAAT_SCRATCH_BYTES per device, created when the library's
 * code loads on that device and held until the process ends; its device address is
 * looked up on the first call on each device.  Returns CAAT_EWORKSPACE when
 * caat_workspace_bytes(handle, T) exceeds CAAT_SCRATCH_BYTES.  Every call on one device
 * shares that device's array: calls that overlap on one device (different streams,
 * handles or threads) race on it and must be serialized by the caller (one stream is
 * enough).  Nothing in it needs clearing between calls. */
int caat_forward_scratch(caat_handle handle, const caat_args *args);

/* Which row-parallel path a forward over T tokens takes: 1 when the shared channels
 * are summed over the ranks inside the GEMM (steps 1 and 2 above, then K3 on S), 0 when
 * every rank's partials are written and K3 sums them; CAAT_EINVAL for a NULL handle or
 * T < 1.  Host only. */
int caat_forward_fused(caat_handle handle, int T);

/* Whether a forward over T tokens that stores out_resid takes the private channels'
 * residual add into the row-parallel GEMM (Eq. 9's r = R + Z on l >= n_s, with Z the
 * rank's own partial, §4 private scaling applied): that GEMM's epilogue writes those
 * columns of out_resid directly (on the per-rank path, from n_s rounded up to a multiple
 * of 8; the chunk that straddles n_s still goes through the partials) and K3 reads them
 * back instead of the partials and the residual.  1 in bf16 for T > 64 where K3's
 * single-pass kernel runs (rows of up to 4096 channels at P = 8; 16384 at P <= 2) and such
 * private columns exist, 0 otherwise (and whenever out_resid is NULL); CAAT_EINVAL for a
 * NULL handle or T < 1.  The outputs meet the same contract either way.  Host only. */
int caat_forward_private_in_epilogue(caat_handle handle, int T);

/* caat_forward_ex that also records caller-created hipEvent_t events[k] on the stream
 * after step k (k < n_events; a NULL entry is skipped), so that a caller can time each
 * step of exactly this call.  The kernels and the results are those of caat_forward_ex.
 * CAAT_EINVAL for n_events < 0, or n_events > 0 with events == NULL. */
int caat_forward_timed(caat_handle handle, const caat_args *args, void *const *events,
                       int n_events);

/* caat_forward_ex for training (MLP only): the same outputs, and preact [P][T][F1]
 * (caller-owned, 16-byte aligned) receives the raw pre-activation x W1^T (SwiGLU: the
 * gate columns [0, f_s), then the up columns), the operand of sigma' in the backward of
 * Eq. 22.  Passed to caat_backward (caat_bwd_args.preact), it replaces the backward's
 * recompute GEMM with bitwise-identical values.  Returns CAAT_EINVAL for CAAT_NONE. */
int caat_forward_train(caat_handle handle, const caat_args *args, void *preact);

/* Step a1 alone (MLP only): Y = act(x W1^T) per rank, x [P][T][h] -> Y [P][T][f_s].
 * First sum of Eq. 22 and the nonlinearity. */
int caat_column_gemm_act(caat_handle handle, int T, const void *x, const void *W1, void *Y,
                         void *stream);

/* Step a2 alone: partials Zt [P][T][h] = in W2^T per rank, in = Y [P][T][f_s] (MLP,
 * second sum of Eq. 22) or H [P][T][h/P] (out-projection, Eq. 24). */
int caat_row_gemm(caat_handle handle, int T, const void *in, const void *W2, void *partials,
                  void *stream);

/* Step a2 with the reduce of step a3 folded in (the paper's single-device local
 * summation, §3.2, done inside the GEMM): the shared channels are summed over the
 * ranks in the GEMM's fp32 accumulators, as one product whose contraction runs over
 * every rank's K (Eq. 22: sum over m of Zt_m[l] for l < n_s):
 *   S [T][n_s]        S[t][l] = sum_m sum_k in_m[t][k] W2_m[l][k],  l < n_s
 *   partials [P][T][h] columns [n_s, h) only: Zt_m[t][l],            l >= n_s
 * Columns [0, n_s) of partials are not written.  S may be NULL when n_s == 0 and
 * partials may be NULL when n_s == h.  Needs n_s % 8 == 0, else CAAT_EUNSUPPORTED.
 * caat_forward / caat_forward_ex take this path when n_s % 8 == 0, T > 64 and the
 * shared-channel GEMM has at least 256 output tiles of 128 x 128, ceil(n_s / 128) x
 * ceil(T / 128) >= 256 (or n_s == 0), unless the concatenated contraction is too long
 * for the kernel's 32-bit offsets (bf16: past 2^31 bytes of P T k2 inputs, where this
 * call returns CAAT_EUNSUPPORTED); caat_forward_fused tells which path a T takes. */
int caat_row_gemm_reduce(caat_handle handle, int T, const void *in, const void *W2, void *S,
                         void *partials, void *stream);

/* Steps a3-a5 after caat_row_gemm_reduce: shared channels from S [T][n_s], private
 * channels from columns [n_s, h) of partials (× s_priv), residual add and
 * normalization (Eq. 9), for every rank.  Same NULL rules and n_s % 8 == 0 rule. */
int caat_sync_norm(caat_handle handle, int T, const void *S, const void *partials,
                   const void *resid, const void *gamma, const void *beta, void *out,
                   void *out_resid, void *stream);

/* Steps a3-a5 alone: partial channel-reduce of the given partials [P][T][h] (Eq. 22 /
 * 24), private scaling, residual add and normalization (Eq. 9).  resid [P][T][h] is
 * required; beta and out_resid may be NULL. */
int caat_partial_sync_norm(caat_handle handle, int T, const void *partials, const void *resid,
                           const void *gamma, const void *beta, void *out, void *out_resid,
                           void *stream);

/* ------------------------------------------------------------------------------
 * Backward of the sublayer: §4 "Forward-backward mismatch" (Eq. 9-13) and App. B
 * (Eq. 25-30).  The loss reaches the sublayer through out (gradient dout) and through
 * the residual stream out_resid = r (gradient dres, from whatever later adds r in).
 * Per rank m and token:
 *   g_m = dres_m + (dNorm/dr at r_m)^T dout_m      (the norm derivative comes first)
 *   dZt_m[l] = sum over ranks q of g_q[l]  for l < n_s   (the reduce after the norm
 *   dZt_m[l] = s_priv * g_m[l]             for l >= n_s   derivative, Eq. 26-28)
 *   dresid_m = g_m
 *   dgamma = sum over ranks and tokens of dout * nhat, dbeta = sum of dout (LayerNorm;
 *   zero for RMSNorm): the norm parameters reduced over ranks (Eq. 12, 29).
 * Then the chain rule through the row-parallel GEMM, the activation and the
 * column-parallel GEMM (Eq. 22 / 24).  The sum over ranks and every contraction
 * accumulate in fp32 (§4: 32-bit accumulation of the reduced gradients); dgamma and
 * dbeta are fp32 outputs, every other tensor is in the handle's dtype.
 * Statistics are recomputed from out_resid as stored by the forward.
 * ------------------------------------------------------------------------------ */

/* Bytes of device workspace caat_backward needs for T tokens (0 for a NULL handle or
 * T < 1).  caat_partial_sync_norm_backward needs 8 * h * min(T, 256) + 512 bytes of it. */
size_t caat_backward_workspace_bytes(caat_handle handle, int T);

typedef struct {
    int T;
    const void *in;         /* the forward's input: x [P][T][h], or H [P][T][h/P] */
    const void *W1;         /* [P][F1][h]; ignored for CAAT_NONE */
    const void *W2;         /* [P][h][k2] */
    const void *gamma;      /* [h] */
    const void *out_resid;  /* r [P][T][h] from the forward (required) */
    const void *dout;       /* dL/d out [P][T][h] */
    const void *dres;       /* dL/d out_resid [P][T][h]; NULL means zero */
    void *din;              /* dL/d in [P][T][h] or [P][T][h/P] */
    void *dresid;           /* dL/d resid [P][T][h]; NULL (MLP only): the forward's
                               residual was `in`, and its gradient is added into din */
    void *dW1;              /* [P][F1][h]; ignored for CAAT_NONE */
    void *dW2;              /* [P][h][k2] */
    float *dgamma;          /* [h], fp32 */
    float *dbeta;           /* [h], fp32, or NULL */
    void *workspace;        /* caller-owned device memory, 16-byte aligned */
    size_t workspace_bytes; /* >= caat_backward_workspace_bytes(T) */
    void *stream;
    void *const *events;    /* NULL, or n_events hipEvent_t: event k is recorded on the
                               stream after step k (see CAAT_BWD_STEPS), for timing */
    int n_events;
    const void *preact;     /* NULL: recompute x W1^T; else the pre-activation
                               caat_forward_train stored [P][T][F1] (MLP only) */
} caat_bwd_args;

/* The steps of caat_backward, in launch order (for caat_bwd_args.events).  Steps that
 * do not apply (CAAT_NONE has no first GEMM) launch nothing; their events are still
 * recorded.
 *   0 norm derivative + reduce over ranks + dgamma/dbeta    1 transpose of W2
 *   2 GEMM dY = dZt W2                                       3 GEMM a = x W1^T (recompute;
 *                                                              nothing when preact is given)
 *   4 activation backward (da, Y)                            5 transpose of W1
 *   6 GEMM dx = da W1 (+ residual gradient when resid = in)  7 transposes of da and x
 *   8 GEMM dW1 = da^T x                                      9 transposes of Y (or H), dZt
 *  10 GEMM dW2 = dZt^T Y
 * With bf16 (and h, k2, F1 multiples of 8) the weight-gradient GEMMs contract over tokens
 * straight from the token-major operands: steps 7 and 9 launch nothing. */
#define CAAT_BWD_STEPS 11

/* The whole backward of one sublayer for every rank.  Returns CAAT_EWORKSPACE for a
 * missing or short workspace, CAAT_EINVAL for bad pointers (a NULL dresid with
 * CAAT_NONE included).  The workspace is overwritten. */
int caat_backward(caat_handle handle, const caat_bwd_args *args);

/* The norm derivative and the reduce over ranks alone (the first step of
 * caat_backward): out_resid, dout [P][T][h], dres (NULL: zero) -> dpartials = dZt
 * [P][T][h], dresid [P][T][h] (NULL: not stored), dgamma [h] and dbeta [h] (NULL: not
 * stored), both fp32. */
int caat_partial_sync_norm_backward(caat_handle handle, int T, const void *out_resid,
                                    const void *dout, const void *dres, const void *gamma,
                                    void *dpartials, void *dresid, float *dgamma, float *dbeta,
                                    void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------------
 * The full block with logical devices (§3.2; App. A.1 Eq. 16 / 18, App. A.2 Eq. 24):
 * per rank m, the QKV projection of the rank's nh heads, causal softmax attention per
 * head, then the out-projection sublayer and the MLP sublayer above.  bf16 only;
 * head width d = 64 or 128.
 * ------------------------------------------------------------------------------ */

/* Bytes of device workspace caat_attention needs (V transposed per head). */
size_t caat_attention_workspace_bytes(int P, int T, int nh, int d);

/* The attention core alone, bf16: for every rank m < P and head i < nh,
 *   H[m][t][i d .. i d + d) = sum over j of softmax_j(q_t . k_j / sqrt(d)) v_j,
 * j running over the tokens of t's sequence up to t (causal).  The T tokens are T / S
 * sequences of S tokens (T % S == 0, S % 8 == 0).
 *   qkv [P][T][3 nh d]: Q of head i in columns [i d, i d + d), K at nh d + i d, V at
 *       2 nh d + i d (the QKV projection's output, rank by rank).
 *   H   [P][T][nh d].
 * d must be 64 or 128 (else CAAT_EUNSUPPORTED). */
int caat_attention(int P, int T, int S, int nh, int d, const void *qkv, void *H,
                   void *workspace, size_t workspace_bytes, void *stream);

typedef struct {
    int T, S;               /* tokens; sequence length (T % S == 0, S % 8 == 0) */
    const void *in;         /* block input h [P][T][h] (the previous block's out) */
    const void *resid;      /* residual stream r [P][T][h] (the previous out_resid) */
    const void *Wqkv;       /* [P][3 h/P][h]: rows [0, h/P) Q, [h/P, 2h/P) K, then V of
                               the rank's heads (row n of shard m = column n of W^{Q|K|V}_m) */
    const void *Wo;         /* [P][h][h/P] (the out-projection's W2) */
    const void *W1, *W2;    /* the MLP's weights, as for caat_forward_ex */
    const void *gamma_attn, *beta_attn, *gamma_mlp, *beta_mlp;  /* [h]; betas may be NULL */
    void *out, *out_resid;  /* [P][T][h]: the next block's in and resid */
    void *workspace;        /* caat_block_workspace_bytes of it */
    size_t workspace_bytes;
    void *stream;
    void *const *events;    /* NULL, or n_events hipEvent_t recorded after each step:
                               0 QKV GEMM, 1 V transpose, 2 attention, 3 out-projection
                               sublayer, 4 MLP sublayer (for timing) */
    int n_events;
} caat_block_args;

/* Bytes of block workspace (QKV, V^T, head outputs and the out-projection sublayer's
 * outputs), 0 if the handles do not form a block: attn must be a CAAT_NONE handle and
 * mlp an MLP handle with the same h, P and norm, both CAAT_BF16, and h/P must split into
 * nh heads of width 64 or 128. */
size_t caat_block_workspace_bytes(caat_handle attn, caat_handle mlp, int nh, int T);

/* One block: QKV projection, attention, out-projection sublayer (residual = resid), MLP
 * sublayer.  The two handles' own workspaces (caat_set_workspace) must also be set for
 * T tokens. */
int caat_block_forward(caat_handle attn, caat_handle mlp, int nh, const caat_block_args *args);

/* Static text for a caat_status. */
const char *caat_error_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* CAAT_H */
