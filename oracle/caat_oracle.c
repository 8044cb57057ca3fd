/*
 * CAAT partial-sync sublayer forward: the ORACLE.
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
