/*
 * CAAT partial-sync sublayer forward and backward: the ORACLE.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, fp64 CPU statement of
 * what one CAAT tensor-parallel sublayer computes.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it.  The GPU library never
 * links, includes or calls it, and it shares no code with the GPU library.
 *
 * Source: "Tensor-Parallelism with Partially Synchronized Activations"
 * (Lamprecht, Karnieli, Hanani, Giladi, Soudry), the arXiv HTML page.
 *
 *   - MLP with partial channel-reduce: App. A.2, Eq. 22 (the P = 2 case is §3.1,
 *     Eq. 6-8).  Each rank m computes its own partial output
 *         zt[m][t][l] = sum_k act( sum_j x[m][t][j] * A[m][j][k] ) * B[m][k][l]
 *     and the channel-reduce sums zt over m only for channels l < floor(h*p).
 *   - Attention output projection with partial channel-reduce: App. A.2, Eq. 24
 *     (P = 2: App. A.1, Eq. 19).  zt[m][t][l] = sum_j H[m][t][j] * O[m][j][l].
 *   - Shared channels are the first h*p channels, fixed at initialization (§3).
 *   - Logical devices: one device computes every rank in turn and replaces the
 *     collective by a local sum (§3.2).  This is the structure of this file.
 *   - Residual add and normalization after the reduce, per rank: §4, Eq. 9, and
 *     App. B, Eq. 25 (the residual splits off before the normalization).
 *   - Private channel scaling by sqrt(r): §4, "Private channel scaling", Eq. 14-15.
 *   - Backward: §4 "Forward-backward mismatch" (Eq. 9-13) and App. B (Eq. 25-30):
 *     the reduce over ranks comes after the norm derivative, and the norm
 *     parameters' gradients are summed over ranks.
 *
 * Readings where the page is silent (each one is listed in the design notes):
 *   - n_s = floor(h*p), where an h*p within 1e-9*h of an integer k counts as k.
 *   - GeLU is the exact erf form unless the tanh form is asked for; SwiGLU is
 *     silu(x A_gate) * (x A_up), with shard m holding the same column range of
 *     A_gate and A_up (rows [0,f_s) gate, [f_s,2f_s) up of the shard).
 *   - Private scaling multiplies the private channels of the reduced output
 *     before the residual add.
 *   - LayerNorm uses the biased (population) variance; RMSNorm divides by
 *     sqrt(mean(r^2) + eps).  No biases and no dropout anywhere.
 *
 * Storage conventions (all row-major, element counts in brackets):
 *   x      [P][T][kin]   kin = h (MLP) or h/P (attention context H_m)
 *   resid  [P][T][h]     NULL means "resid = x" (MLP only, kin == h)
 *   W1     [P][F1][h]    F1 = f_s (GeLU) or 2*f_s (SwiGLU); row k of shard m is
 *                        column k of A_m (so the contraction runs along a row)
 *   W2     [P][h][k2]    k2 = f_s (MLP) or h/P (attention); row l of shard m is
 *                        column l of B_m (or O_m)
 *   gamma, beta [h]      shared by all ranks; beta NULL means zero
 * Inputs are float32 (exact for bf16 and fp32 values); all arithmetic is fp64.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_GELU = 0, ORACLE_GELU_TANH = 1, ORACLE_SWIGLU = 2, ORACLE_NONE = 3 };
enum { ORACLE_LAYERNORM = 0, ORACLE_RMSNORM = 1 };

/* Threads the OpenMP loops below use. */
int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Number of shared channels (§3: "the first h*p channels"; App. A.2, Eq. 22:
 * channel l is reduced iff l < floor(h p)).  An h*p that fp64 puts a hair below an
 * integer (100 * 0.29 = 28.999999999999996) counts as that integer. */
int oracle_shared_channels(int h, double p)
{
    double hp = (double)h * p;
    double k = nearbyint(hp);
    if (fabs(hp - k) <= 1e-9 * (double)h)
        return (int)k;
    return (int)floor(hp);
}

/* The nonlinearity sigma of Eq. 20-22.  GeLU (exact): a * Phi(a), Phi the standard
 * normal CDF.  GeLU (tanh
 * form): the approximation published with GeLU by Hendrycks and Gimpel.  SwiGLU:
 * silu(g) * u with silu(g) = g / (1 + e^-g).  NONE: identity (no first layer). */
double oracle_activation(int act, double g, double u)
{
    switch (act) {
    case ORACLE_GELU:
        /* a * Phi(a), with Phi(a) = erfc(-a / sqrt 2) / 2 (no cancellation for a < 0) */
        return 0.5 * g * erfc(-g / sqrt(2.0));
    case ORACLE_GELU_TANH: {
        const double c = sqrt(2.0 / 3.14159265358979323846);
        return 0.5 * g * (1.0 + tanh(c * (g + 0.044715 * g * g * g)));
    }
    case ORACLE_SWIGLU:
        return g / (1.0 + exp(-g)) * u;
    default:
        return g;
    }
}

/* One rank's partial output row zt[m][t][:] before any reduction (the tilde
 * quantity of Eq. 22 / Eq. 24).  y is scratch of at least max(f_s, kin) doubles. */
static void rank_partial_row(int act, int h, int fs, int kin,
                             const float *x_row, const float *W1m, const float *W2m,
                             double *y, double *zt_row)
{
    int k2;
    if (act == ORACLE_NONE) {
        /* Attention out-projection: the input row is the head output H_m (Eq. 24). */
        for (int j = 0; j < kin; ++j)
            y[j] = (double)x_row[j];
        k2 = kin;
    } else {
        /* First sum of Eq. 22: a_k = sum_j x_j A_jk, then the nonlinearity. */
        for (int k = 0; k < fs; ++k) {
            double a = 0.0;
            for (int j = 0; j < h; ++j)
                a += (double)x_row[j] * (double)W1m[(size_t)k * h + j];
            double u = 0.0;
            if (act == ORACLE_SWIGLU) {
                for (int j = 0; j < h; ++j)
                    u += (double)x_row[j] * (double)W1m[(size_t)(fs + k) * h + j];
            }
            y[k] = oracle_activation(act, a, u);
        }
        k2 = fs;
    }
    /* Second sum of Eq. 22 (or the sum over j of Eq. 24): zt_l = sum_k y_k B_kl. */
    for (int l = 0; l < h; ++l) {
        double z = 0.0;
        for (int k = 0; k < k2; ++k)
            z += y[k] * (double)W2m[(size_t)l * k2 + k];
        zt_row[l] = z;
    }
}

/* Partial channel-reduce (Eq. 22 / 24), private scaling (§4), residual add and
 * normalization (Eq. 9) for every rank m and token t.
 * zt [P][T][h] fp64; resid [P][T][h] float; out, out_resid [P][T][h] fp64. */
static void reduce_residual_norm(int P, int T, int h, int n_s, double s_priv, double eps,
                                 int norm, const double *zt, const float *resid,
                                 const float *gamma, const float *beta,
                                 double *out, double *out_resid)
{
#pragma omp parallel
    {
        double *S = (double *)malloc(sizeof(double) * (size_t)(n_s > 0 ? n_s : 1));
        double *r = (double *)malloc(sizeof(double) * (size_t)h);
#pragma omp for schedule(static)
        for (int t = 0; t < T; ++t) {
            /* Shared channels: sum over all ranks (the partial channel-reduce). */
            for (int l = 0; l < n_s; ++l) {
                double s = 0.0;
                for (int m = 0; m < P; ++m)
                    s += zt[((size_t)m * T + t) * h + l];
                S[l] = s;
            }
            for (int m = 0; m < P; ++m) {
                size_t row = ((size_t)m * T + t) * h;
                /* Z_m: reduced value on shared channels, own (scaled) value on
                 * private channels; then the per-rank residual add. */
                for (int l = 0; l < h; ++l) {
                    double z = (l < n_s) ? S[l] : s_priv * zt[row + l];
                    r[l] = (double)resid[row + l] + z;
                }
                double inv;
                double mean = 0.0;
                if (norm == ORACLE_LAYERNORM) {
                    for (int l = 0; l < h; ++l)
                        mean += r[l];
                    mean /= (double)h;
                    double var = 0.0;
                    for (int l = 0; l < h; ++l)
                        var += (r[l] - mean) * (r[l] - mean);
                    var /= (double)h;
                    inv = 1.0 / sqrt(var + eps);
                } else {
                    double ms = 0.0;
                    for (int l = 0; l < h; ++l)
                        ms += r[l] * r[l];
                    ms /= (double)h;
                    inv = 1.0 / sqrt(ms + eps);
                }
                for (int l = 0; l < h; ++l) {
                    double b = (norm == ORACLE_LAYERNORM && beta) ? (double)beta[l] : 0.0;
                    out[row + l] = (r[l] - mean) * inv * (double)gamma[l] + b;
                    if (out_resid)
                        out_resid[row + l] = r[l];
                }
            }
        }
        free(S);
        free(r);
    }
}

static int check_common(int P, int T, int h, int n_s, int norm)
{
    if (P < 1 || T < 0 || h < 1 || n_s < 0 || n_s > h)
        return -1;
    if (norm != ORACLE_LAYERNORM && norm != ORACLE_RMSNORM)
        return -1;
    return 0;
}

/* Full sublayer forward for T token rows (any subset of a larger batch: token rows
 * do not interact).  zt_out [P][T][h] may be NULL.  Returns 0, or -1 on bad args. */
int oracle_sublayer(int P, int T, int h, int ffn, int act, int norm, int n_s,
                    double s_priv, double eps,
                    const float *x, const float *resid, const float *W1, const float *W2,
                    const float *gamma, const float *beta,
                    double *zt_out, double *out, double *out_resid)
{
    if (check_common(P, T, h, n_s, norm))
        return -1;
    if (act < ORACLE_GELU || act > ORACLE_NONE)
        return -1;
    int fs = 0, kin, F1 = 0;
    if (act == ORACLE_NONE) {
        if (h % P)
            return -1;
        kin = h / P;
    } else {
        if (ffn % P)
            return -1;
        fs = ffn / P;
        F1 = (act == ORACLE_SWIGLU) ? 2 * fs : fs;
        kin = h;
    }
    if (resid == NULL) {
        if (act == ORACLE_NONE)
            return -1;
        resid = x;
    }
    int k2 = (act == ORACLE_NONE) ? kin : fs;
    double *zt = zt_out ? zt_out : (double *)malloc(sizeof(double) * (size_t)P * T * h + 8);
    if (!zt)
        return -1;

    /* Logical devices (§3.2): every rank's layer output, one rank after another. */
#pragma omp parallel
    {
        int ylen = fs > kin ? fs : kin;
        double *y = (double *)malloc(sizeof(double) * (size_t)(ylen > 0 ? ylen : 1));
#pragma omp for collapse(2) schedule(static)
        for (int m = 0; m < P; ++m)
            for (int t = 0; t < T; ++t) {
                const float *x_row = x + ((size_t)m * T + t) * kin;
                const float *W1m = (act == ORACLE_NONE) ? NULL : W1 + (size_t)m * F1 * h;
                const float *W2m = W2 + (size_t)m * h * k2;
                rank_partial_row(act, h, fs, kin, x_row, W1m, W2m, y,
                                 zt + ((size_t)m * T + t) * h);
            }
        free(y);
    }

    reduce_residual_norm(P, T, h, n_s, s_priv, eps, norm, zt, resid, gamma, beta,
                         out, out_resid);
    if (!zt_out)
        free(zt);
    return 0;
}

/* The reduce + residual + norm step alone, on given partials zt [P][T][h] (float). */
int oracle_partial_sync_norm(int P, int T, int h, int norm, int n_s, double s_priv, double eps,
                             const float *partials, const float *resid,
                             const float *gamma, const float *beta,
                             double *out, double *out_resid)
{
    if (check_common(P, T, h, n_s, norm))
        return -1;
    size_t n = (size_t)P * T * h;
    double *zt = (double *)malloc(sizeof(double) * n + 8);
    if (!zt)
        return -1;
    for (size_t i = 0; i < n; ++i)
        zt[i] = (double)partials[i];
    reduce_residual_norm(P, T, h, n_s, s_priv, eps, norm, zt, resid, gamma, beta,
                         out, out_resid);
    free(zt);
    return 0;
}

/* ---------------------------------------------------------------------------------
 * Backward of the sublayer (§4 "Forward-backward mismatch", Eq. 9-13; App. B,
 * Eq. 25-30).  The loss reaches the sublayer through out = Norm(r) (upstream
 * gradient dout) and through the residual stream r itself (upstream gradient dres,
 * the gradient of whatever the next sublayer adds r into).  Per rank m:
 *   g_m = dres_m + (dNorm/dr at r_m)^T dout_m      -- the norm derivative first, per
 *                                                   rank (the 'h' placement of §4)
 *   dZt_q[l] = sum_m g_m[l]      for l < n_s      -- the reduce after the norm
 *   dZt_q[l] = s_priv * g_q[l]   for l >= n_s        derivative (Eq. 26-28)
 *   dresid_m = g_m                                   (the residual term of Eq. 26)
 *   dgamma = sum_{m,t} dout * nhat, dbeta = sum_{m,t} dout   (Eq. 12, 29: the norm
 *                                                   parameters reduced over ranks)
 * then the chain rule through the two GEMMs and the nonlinearity of Eq. 22 / 24.
 */

/* d sigma / d a for the one-input activations (GeLU forms). */
static double act_grad(int act, double a)
{
    if (act == ORACLE_GELU) {
        /* d/da [a Phi(a)] = Phi(a) + a phi(a) */
        const double Phi = 0.5 * erfc(-a / sqrt(2.0));
        const double phi = exp(-0.5 * a * a) / sqrt(2.0 * 3.14159265358979323846);
        return Phi + a * phi;
    }
    if (act == ORACLE_GELU_TANH) {
        const double c = sqrt(2.0 / 3.14159265358979323846);
        const double u = c * (a + 0.044715 * a * a * a);
        const double th = tanh(u);
        return 0.5 * (1.0 + th) + 0.5 * a * (1.0 - th * th) * c * (1.0 + 3.0 * 0.044715 * a * a);
    }
    return 1.0;
}

/* Returns 0, or -1 on bad arguments.  Outputs (fp64, all overwritten):
 *   dx     [P][T][kin]  gradient of the loss w.r.t. x (when resid is NULL, i.e.
 *                       resid = x, the residual gradient is included)
 *   dresid [P][T][h]    gradient w.r.t. resid (may be NULL)
 *   dW1    [P][F1][h]   (NULL for act = NONE), dW2 [P][h][k2]
 *   dgamma [h], dbeta [h] (dbeta is zero for RMSNorm)
 * dres NULL means zero.  zt and the norm statistics are recomputed here. */
int oracle_sublayer_backward(int P, int T, int h, int ffn, int act, int norm, int n_s,
                             double s_priv, double eps,
                             const float *x, const float *resid, const float *W1,
                             const float *W2, const float *gamma,
                             const float *dout, const float *dres,
                             double *dx, double *dresid, double *dW1, double *dW2,
                             double *dgamma, double *dbeta)
{
    if (check_common(P, T, h, n_s, norm) || act < ORACLE_GELU || act > ORACLE_NONE)
        return -1;
    int fs = 0, kin, F1 = 0;
    if (act == ORACLE_NONE) {
        if (h % P)
            return -1;
        kin = h / P;
    } else {
        if (ffn % P)
            return -1;
        fs = ffn / P;
        F1 = (act == ORACLE_SWIGLU) ? 2 * fs : fs;
        kin = h;
    }
    const int resid_is_x = (resid == NULL);
    if (resid_is_x) {
        if (act == ORACLE_NONE)
            return -1;
        resid = x;
    }
    const int k2 = (act == ORACLE_NONE) ? kin : fs;
    const size_t rows = (size_t)P * T;
    double *a = (double *)calloc(rows * (size_t)(F1 > 0 ? F1 : 1), sizeof(double));
    double *y = (double *)calloc(rows * (size_t)k2, sizeof(double));
    double *zt = (double *)calloc(rows * (size_t)h, sizeof(double));
    double *nh = (double *)calloc(rows * (size_t)h, sizeof(double));
    double *g = (double *)calloc(rows * (size_t)h, sizeof(double));
    double *dzt = (double *)calloc(rows * (size_t)h, sizeof(double));
    double *da = (double *)calloc(rows * (size_t)(F1 > 0 ? F1 : 1), sizeof(double));
    if (!a || !y || !zt || !nh || !g || !dzt || !da) {
        free(a); free(y); free(zt); free(nh); free(g); free(dzt); free(da);
        return -1;
    }

    /* Forward recompute: pre-activations a, activations y (the GEMM-2 input) and the
     * partials zt of every rank (Eq. 22 / 24). */
#pragma omp parallel for collapse(2) schedule(static)
    for (int m = 0; m < P; ++m)
        for (int t = 0; t < T; ++t) {
            const size_t row = (size_t)m * T + t;
            const float *xr = x + row * kin;
            double *ar = a + row * (size_t)(F1 > 0 ? F1 : 1), *yr = y + row * k2;
            if (act == ORACLE_NONE) {
                for (int j = 0; j < kin; ++j)
                    yr[j] = (double)xr[j];
            } else {
                const float *W1m = W1 + (size_t)m * F1 * h;
                for (int k = 0; k < F1; ++k) {
                    double s = 0.0;
                    for (int j = 0; j < h; ++j)
                        s += (double)xr[j] * (double)W1m[(size_t)k * h + j];
                    ar[k] = s;
                }
                for (int k = 0; k < fs; ++k)
                    yr[k] = oracle_activation(act, ar[k], act == ORACLE_SWIGLU ? ar[fs + k] : 0.0);
            }
            const float *W2m = W2 + (size_t)m * h * k2;
            for (int l = 0; l < h; ++l) {
                double s = 0.0;
                for (int k = 0; k < k2; ++k)
                    s += yr[k] * (double)W2m[(size_t)l * k2 + k];
                zt[row * h + l] = s;
            }
        }

    /* Per token: forward reduce + residual + statistics, then the norm derivative of
     * every rank (before any reduction), then the backward reduce. */
#pragma omp parallel
    {
        double *r = (double *)malloc(sizeof(double) * (size_t)h);
#pragma omp for schedule(static)
        for (int t = 0; t < T; ++t) {
            for (int m = 0; m < P; ++m) {
                const size_t row = ((size_t)m * T + t) * h;
                for (int l = 0; l < h; ++l) {
                    double z;
                    if (l < n_s) {
                        z = 0.0;
                        for (int q = 0; q < P; ++q)
                            z += zt[((size_t)q * T + t) * h + l];
                    } else {
                        z = s_priv * zt[row + l];
                    }
                    r[l] = (double)resid[row + l] + z;
                }
                double mean = 0.0, inv;
                if (norm == ORACLE_LAYERNORM) {
                    for (int l = 0; l < h; ++l)
                        mean += r[l];
                    mean /= (double)h;
                    double var = 0.0;
                    for (int l = 0; l < h; ++l)
                        var += (r[l] - mean) * (r[l] - mean);
                    inv = 1.0 / sqrt(var / (double)h + eps);
                } else {
                    double ms = 0.0;
                    for (int l = 0; l < h; ++l)
                        ms += r[l] * r[l];
                    inv = 1.0 / sqrt(ms / (double)h + eps);
                }
                /* nhat = (r - mean) inv; dnhat = dout * gamma;
                 * LN:  dr = inv (dnhat - mean(dnhat) - nhat mean(dnhat nhat))
                 * RMS: dr = inv (dnhat - nhat mean(dnhat nhat)) */
                double s1 = 0.0, s2 = 0.0;
                for (int l = 0; l < h; ++l) {
                    const double n = (r[l] - mean) * inv;
                    const double dn = (double)dout[row + l] * (double)gamma[l];
                    nh[row + l] = n;
                    s1 += dn;
                    s2 += dn * n;
                }
                s1 /= (double)h;
                s2 /= (double)h;
                for (int l = 0; l < h; ++l) {
                    const double dn = (double)dout[row + l] * (double)gamma[l];
                    double dr = dn - nh[row + l] * s2;
                    if (norm == ORACLE_LAYERNORM)
                        dr -= s1;
                    g[row + l] = inv * dr + (dres ? (double)dres[row + l] : 0.0);
                }
            }
            /* The reduce after the norm derivative: shared channels of every rank's
             * partial receive the sum over ranks of g; private ones their own g. */
            for (int m = 0; m < P; ++m) {
                const size_t row = ((size_t)m * T + t) * h;
                for (int l = 0; l < h; ++l) {
                    double d;
                    if (l < n_s) {
                        d = 0.0;
                        for (int q = 0; q < P; ++q)
                            d += g[((size_t)q * T + t) * h + l];
                    } else {
                        d = s_priv * g[row + l];
                    }
                    dzt[row + l] = d;
                }
            }
        }
        free(r);
    }

    /* Norm parameters: summed over ranks and tokens (Eq. 12, 29). */
#pragma omp parallel for schedule(static)
    for (int l = 0; l < h; ++l) {
        double sg = 0.0, sb = 0.0;
        for (size_t row = 0; row < rows; ++row) {
            sg += (double)dout[row * h + l] * nh[row * h + l];
            sb += (double)dout[row * h + l];
        }
        dgamma[l] = sg;
        dbeta[l] = (norm == ORACLE_LAYERNORM) ? sb : 0.0;
    }

    /* Second GEMM (Eq. 22 second sum / Eq. 24): dW2 = dzt^T y, dy = dzt W2; then the
     * nonlinearity and the first GEMM: da = dy * sigma'(a), dW1 = da^T x, dx = da W1. */
#pragma omp parallel for collapse(2) schedule(static)
    for (int m = 0; m < P; ++m)
        for (int l = 0; l < h; ++l)
            for (int k = 0; k < k2; ++k) {
                double s = 0.0;
                for (int t = 0; t < T; ++t) {
                    const size_t row = (size_t)m * T + t;
                    s += dzt[row * h + l] * y[row * k2 + k];
                }
                dW2[((size_t)m * h + l) * k2 + k] = s;
            }
#pragma omp parallel
    {
        double *dy = (double *)malloc(sizeof(double) * (size_t)(k2 > 0 ? k2 : 1));
#pragma omp for collapse(2) schedule(static)
        for (int m = 0; m < P; ++m)
            for (int t = 0; t < T; ++t) {
                const size_t row = (size_t)m * T + t;
                const float *W2m = W2 + (size_t)m * h * k2;
                for (int k = 0; k < k2; ++k) {
                    double s = 0.0;
                    for (int l = 0; l < h; ++l)
                        s += dzt[row * h + l] * (double)W2m[(size_t)l * k2 + k];
                    dy[k] = s;
                }
                if (act == ORACLE_NONE) {
                    for (int j = 0; j < kin; ++j)
                        dx[row * kin + j] = dy[j];
                    continue;
                }
                double *ar = a + row * F1, *dar = da + row * F1;
                for (int k = 0; k < fs; ++k) {
                    if (act == ORACLE_SWIGLU) {
                        /* y = silu(g) u: dg = dy u silu'(g), du = dy silu(g),
                         * silu'(g) = sig(g) (1 + g (1 - sig(g))) */
                        const double gg = ar[k], uu = ar[fs + k];
                        const double sg = 1.0 / (1.0 + exp(-gg));
                        dar[k] = dy[k] * uu * sg * (1.0 + gg * (1.0 - sg));
                        dar[fs + k] = dy[k] * gg * sg;
                    } else {
                        dar[k] = dy[k] * act_grad(act, ar[k]);
                    }
                }
                const float *W1m = W1 + (size_t)m * F1 * h;
                for (int j = 0; j < h; ++j) {
                    double s = 0.0;
                    for (int k = 0; k < F1; ++k)
                        s += dar[k] * (double)W1m[(size_t)k * h + j];
                    dx[row * kin + j] = s + (resid_is_x ? g[row * h + j] : 0.0);
                }
            }
        free(dy);
    }
    if (act != ORACLE_NONE) {
#pragma omp parallel for collapse(2) schedule(static)
        for (int m = 0; m < P; ++m)
            for (int k = 0; k < F1; ++k)
                for (int j = 0; j < h; ++j) {
                    double s = 0.0;
                    for (int t = 0; t < T; ++t) {
                        const size_t row = (size_t)m * T + t;
                        s += da[row * F1 + k] * (double)x[row * kin + j];
                    }
                    dW1[((size_t)m * F1 + k) * h + j] = s;
                }
    }
    if (dresid)
        memcpy(dresid, g, sizeof(double) * rows * (size_t)h);
    free(a); free(y); free(zt); free(nh); free(g); free(dzt); free(da);
    return 0;
}

/* ---------------------------------------------------------------------------------
 * The steps either side of the path, for the full block with logical devices
 * (§3.2; App. A, Eq. 16, 18 and 24).
 */

/* One linear layer per rank: out[m][t][n] = sum_k x[m][t][k] W[m][n][k] (row n of W is
 * the weight column of output n), fp64.  Returns 0, or -1 on bad arguments. */
int oracle_linear(int P, int T, int K, int N, const float *x, const float *W, double *out)
{
    if (P < 1 || T < 0 || K < 1 || N < 1)
        return -1;
#pragma omp parallel for collapse(2) schedule(static)
    for (int m = 0; m < P; ++m)
        for (int t = 0; t < T; ++t) {
            const float *xr = x + ((size_t)m * T + t) * K;
            const float *Wm = W + (size_t)m * N * K;
            double *o = out + ((size_t)m * T + t) * N;
            for (int n = 0; n < N; ++n) {
                double s = 0.0;
                for (int k = 0; k < K; ++k)
                    s += (double)xr[k] * (double)Wm[(size_t)n * K + k];
                o[n] = s;
            }
        }
    return 0;
}

/* Causal self-attention of every head of every rank: H_m = Attention(X_m W^Q_m,
 * X_m W^K_m, X_m W^V_m) (App. A.1 Eq. 16 / 18, App. A.2 Eq. 24), each rank holding nh
 * heads of width d.  qkv [P][T][3 nh d]: per rank and token, Q of head i in columns
 * [i d, (i+1) d), K of head i at nh d + i d, V of head i at 2 nh d + i d.  The T tokens
 * are nseq = T / S sequences of S tokens; token i attends to the tokens j <= i of its
 * own sequence with weights softmax_j(q_i . k_j / sqrt(d)).  H [P][T][nh d] (fp64),
 * head i in columns [i d, (i+1) d).  Returns 0, or -1 on bad arguments. */
int oracle_attention(int P, int T, int S, int nh, int d, const float *qkv, double *H)
{
    if (P < 1 || T < 0 || S < 1 || T % S != 0 || nh < 1 || d < 1)
        return -1;
    const size_t ld = (size_t)3 * nh * d;
    const double scale = 1.0 / sqrt((double)d);
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)S);
#pragma omp for collapse(3) schedule(dynamic, 4)
        for (int m = 0; m < P; ++m)
            for (int hd = 0; hd < nh; ++hd)
                for (int t = 0; t < T; ++t) {
                    const int s0 = (t / S) * S;           /* first token of t's sequence */
                    const float *q = qkv + ((size_t)m * T + t) * ld + (size_t)hd * d;
                    double mx = -INFINITY;
                    for (int j = s0; j <= t; ++j) {
                        const float *k = qkv + ((size_t)m * T + j) * ld + (size_t)(nh + hd) * d;
                        double s = 0.0;
                        for (int e = 0; e < d; ++e)
                            s += (double)q[e] * (double)k[e];
                        w[j - s0] = s * scale;
                        if (w[j - s0] > mx)
                            mx = w[j - s0];
                    }
                    double den = 0.0;
                    for (int j = s0; j <= t; ++j) {
                        w[j - s0] = exp(w[j - s0] - mx);
                        den += w[j - s0];
                    }
                    double *o = H + ((size_t)m * T + t) * (size_t)nh * d + (size_t)hd * d;
                    for (int e = 0; e < d; ++e)
                        o[e] = 0.0;
                    for (int j = s0; j <= t; ++j) {
                        const float *v = qkv + ((size_t)m * T + j) * ld + (size_t)(2 * nh + hd) * d;
                        const double pj = w[j - s0] / den;
                        for (int e = 0; e < d; ++e)
                            o[e] += pj * (double)v[e];
                    }
                }
        free(w);
    }
    return 0;
}
