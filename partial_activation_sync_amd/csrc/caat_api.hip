// libcaat: the C ABI (include/caat.h).  Argument checks, the shared-channel count,
// workspace sizing, the device check and the launch sequence K1 -> K2 -> K3 on the
// caller's stream.  No host synchronisation and no device allocation happen here.
//
// "Tensor-Parallelism with Partially Synchronized Activations": the sublayer is
// App. A.2, Eq. 22 (MLP) / Eq. 24 (attention out-projection), followed by §4, Eq. 9
// (residual + normalization), with every rank on one device (§3.2, logical devices).
#include <math.h>
#include <mutex>
#include <new>
#include <stdlib.h>
#include <string.h>

#include "caat_internal.h"

#define CAAT_API extern "C" __attribute__((visibility("default")))

// The static workspace of caat_forward_scratch, for callers that cannot allocate: one
// copy per device, held until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory, so its device address is looked up once per device (with
// that device current, scratch_address below) and only that address is ever handed to a
// kernel.
static __device__ __align__(256) unsigned char scratch[CAAT_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
int g_arch_ok[MAX_DEVICES];  // 0 unknown, 1 gfx950, -1 other

// Whether the current device is gfx950; cached per device ordinal.  Two host-side test
// hooks come first, read from the environment on every call before any HIP call, so that
// the error paths can be driven without a fault on the GPU:
//   CAAT_FAULT=launch   the call fails as a failed launch does (CAAT_EDEVICE), having
//                       enqueued nothing;
//   CAAT_ARCH=<name>    the device is taken to be that architecture: anything but gfx950
//                       gives CAAT_EUNSUPPORTED (gfx950 falls through to the real query).
int device_check() {
    const char *fault = getenv("CAAT_FAULT");
    if (fault != nullptr && strcmp(fault, "launch") == 0) return CAAT_EDEVICE;
    const char *arch = getenv("CAAT_ARCH");
    if (arch != nullptr && arch[0] != '\0' && strncmp(arch, "gfx950", 6) != 0)
        return CAAT_EUNSUPPORTED;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return CAAT_EDEVICE;
    if (dev < 0 || dev >= MAX_DEVICES) return CAAT_EUNSUPPORTED;
    if (g_arch_ok[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return CAAT_EDEVICE;
        g_arch_ok[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    }
    return g_arch_ok[dev] == 1 ? CAAT_OK : CAAT_EUNSUPPORTED;
}

bool aligned16(const void *p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }
bool aligned16_or_null(const void *p) { return ((uintptr_t)p & 15u) == 0; }

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

size_t esize(const caat_ctx *c) { return c->dtype == CAAT_BF16 ? 2 : 4; }

size_t y_bytes(const caat_ctx *c, int T) {
    return c->act == CAAT_NONE ? 0 : align256((size_t)c->P * T * c->fs * esize(c));
}
size_t partial_bytes(const caat_ctx *c, int T) {
    return align256((size_t)c->P * T * c->h * esize(c));
}
// The fused path (shared channels reduced inside the row-parallel GEMM) needs the
// shared/private boundary on a 16-byte boundary of every row.
bool fused_ok(const caat_ctx *c) { return c->n_s % 8 == 0; }
// caat_forward_ex takes it for prefill-sized batches, where it saves the partials'
// shared columns of every rank (T x n_s x (P - 1) values written and read).  Decode
// batches (T <= 64) keep the per-rank GEMM: their partials are a few MB, and the
// single shared GEMM would spread its weight stream over too few workgroups.
size_t s_bytes(const caat_ctx *c, int T) {
    return fused_ok(c) ? align256((size_t)T * c->n_s * esize(c)) : 0;
}

// Shared channels (§3: the first h p channels; Eq. 22: l < floor(h p)).  An h p that
// lands a rounding error below an integer counts as that integer.
int shared_count(int h, double p) {
    const double hp = (double)h * p;
    const double k = nearbyint(hp);
    if (fabs(hp - k) <= 1e-9 * (double)h) return (int)k;
    return (int)floor(hp);
}

caat::GemmArgs col_args(const caat_ctx *c, int T, const void *x, const void *W1, void *Y) {
    caat::GemmArgs g{};
    g.P = c->P; g.N = c->fs; g.T = T; g.K = c->h;
    g.W = W1; g.w_stride = (size_t)c->F1 * c->h;
    g.X = x;  g.x_stride = (size_t)T * c->h;
    g.out = Y; g.o_stride = (size_t)T * c->fs; g.ldo = c->fs;
    g.up_off = c->fs;
    g.kseg = 1;
    switch (c->act) {
    case CAAT_GELU: g.epi = caat::EPI_GELU; break;
    case CAAT_GELU_TANH: g.epi = caat::EPI_GELU_TANH; break;
    default: g.epi = caat::EPI_SWIGLU; break;
    }
    return g;
}

// The raw pre-activation as one plain GEMM: a[m][t][n] = sum_j x[m][t][j] W1[m][n][j],
// n < F1 (SwiGLU: gate rows, then up rows), row stride F1.
caat::GemmArgs preact_args(const caat_ctx *c, int T, const void *W1, const void *x, void *a) {
    caat::GemmArgs g{};
    g.P = c->P; g.N = c->F1; g.T = T; g.K = c->h;
    g.W = W1; g.w_stride = (size_t)c->F1 * c->h;
    g.X = x;  g.x_stride = (size_t)T * c->h;
    g.out = a; g.o_stride = (size_t)T * c->F1; g.ldo = c->F1;
    g.epi = caat::EPI_STORE;
    g.kseg = 1;
    return g;
}

caat::GemmArgs row_args(const caat_ctx *c, int T, const void *in, const void *W2, void *Z) {
    caat::GemmArgs g{};
    g.P = c->P; g.N = c->h; g.T = T; g.K = c->k2;
    g.W = W2; g.w_stride = (size_t)c->h * c->k2;
    g.X = in; g.x_stride = (size_t)T * c->k2;
    g.out = Z; g.o_stride = (size_t)T * c->h; g.ldo = c->h;
    g.up_off = 0;
    g.epi = caat::EPI_STORE;
    g.kseg = 1;
    return g;
}

// Shared channels [0, n_s): one GEMM whose contraction runs over every rank's K
// (the ranks' partial products summed in the accumulators): S[t][l] =
// sum_m sum_k in_m[t][k] W2_m[l][k], written once, [T][n_s].
caat::GemmArgs shared_args(const caat_ctx *c, int T, const void *in, const void *W2, void *S) {
    caat::GemmArgs g{};
    g.P = 1; g.N = c->n_s; g.T = T; g.K = c->k2;
    g.W = W2; g.w_stride = 0;
    g.X = in; g.x_stride = 0;
    g.out = S; g.o_stride = 0; g.ldo = c->n_s;
    g.up_off = 0;
    g.epi = caat::EPI_STORE;
    g.kseg = c->P; g.w_kseg = (size_t)c->h * c->k2; g.x_kseg = (size_t)T * c->k2;
    return g;
}

// Private channels [n_s, h): the per-rank partials, written into columns [n_s, h) of
// partials[m][t][:].
caat::GemmArgs private_args(const caat_ctx *c, int T, const void *in, const void *W2, void *Z) {
    caat::GemmArgs g = row_args(c, T, in, W2, Z);
    g.N = c->h - c->n_s;
    g.W = reinterpret_cast<const char *>(W2) + (size_t)c->n_s * c->k2 * esize(c);
    g.out = reinterpret_cast<char *>(Z) + (size_t)c->n_s * esize(c);
    return g;
}

// The private channels straight into the residual output (bf16): the private GEMM's
// epilogue writes out_resid[m][t][l] = resid[m][t][l] + s_priv * Zt_m[t][l] for l >= n_s
// (Zt rounded to bf16 first, one fused multiply-add: what K3 computes from the stored
// partials), so the private partials never go through memory and K3 reads those rows
// once instead of the partials and the residual, and writes only the shared columns of
// out_resid.  Per sublayer that removes a [P][T][h - n_s] round trip.
caat::GemmArgs private_resid_args(const caat_ctx *c, int T, const void *in, const void *W2,
                                  const void *resid, void *out_resid) {
    caat::GemmArgs g = private_args(c, T, in, W2, out_resid);
    g.epi = caat::EPI_RESID;
    g.split = 0;
    g.out2 = g.out;
    g.res = reinterpret_cast<const char *>(resid) + (size_t)c->n_s * esize(c);
    g.s_res = c->s_priv;
    return g;
}

// The per-rank row GEMM with the same treatment of the private channels: columns below
// n_s rounded up to 8 are written to the partials (K3 sums their shared channels over
// the ranks; a chunk that straddles n_s goes there whole), the rest straight into
// out_resid as R + s_priv * Zt.
caat::GemmArgs row_resid_args(const caat_ctx *c, int T, const void *in, const void *W2, void *Z,
                              const void *resid, void *out_resid) {
    caat::GemmArgs g = row_args(c, T, in, W2, Z);
    g.epi = caat::EPI_RESID_SPLIT;
    g.split = (c->n_s + 7) / 8 * 8;
    g.out2 = out_resid;
    g.res = resid;
    g.s_res = c->s_priv;
    return g;
}

int run_gemm(const caat_ctx *c, const caat::GemmArgs &g, hipStream_t s);

// Whether caat_forward_ex sums the shared channels inside the row-parallel GEMM.  The
// fused path saves writing and reading the shared columns of P - 1 ranks, but its
// shared-channel GEMM has only ceil(n_s / 128) x ceil(T / 128) output tiles of 128 x 128,
// each contracting over P k2: with fewer tiles than the 256 compute units it leaves CUs
// idle and runs slower than the per-rank GEMM, whose P-fold more tiles split that
// contraction rank by rank (K3 then sums the ranks).  Measured on the 130M pair
// (n_s = 384, T = 4096: 96 tiles): row GEMM 52 against 26 us for the MLP, 18 against
// 12 us for the out-projection; on the 1.1B MLP at p = 0.5 (512 tiles) the fused one
// is faster, 183 against 208 us.  Decode batches (T <= 64) and n_s % 8 != 0 always take
// the per-rank path.  The K-concatenated GEMM must also stay within the bf16 kernel's
// 32-bit byte offsets (its X span is P T k2 elements).
constexpr long FUSED_MIN_TILES = 256;

bool fused_for(const caat_ctx *c, int T) {
    if (!fused_ok(c) || T <= 64) return false;
    if (c->n_s == 0) return true;   // no shared GEMM: the private one is the per-rank GEMM
    const long tiles = (long)((c->n_s + 127) / 128) * ((T + 127) / 128);
    if (tiles < FUSED_MIN_TILES) return false;
    if (c->dtype == CAAT_BF16 &&
        !caat::gemm_bf16_supported(shared_args(c, T, nullptr, nullptr, nullptr)))
        return false;
    return true;
}

// Whether a forward with a residual output writes the private channels' rows from the
// row GEMM's epilogue (bf16, T > 64, K3's single-pass kernel, which reads them, runs, and
// some private channel chunk is left: from n_s on when fused, else from n_s rounded up to
// a whole chunk of 8).
// On the per-rank path only for rows of at least 2^25 elements over all ranks: there the
// bytes K3 saves outweigh the addend the GEMM's epilogue reads (1.1B MLP at p = 0.37,
// T = 8192: 0.741 -> 0.726 ms per replayed step), while the 130M pair (2^23.6) went
// 0.1225 -> 0.1240 ms, its short-K row GEMMs taking what K3 gave back.
constexpr long PER_RANK_DIRECT_MIN = 1L << 25;

bool private_direct_for(const caat_ctx *c, int T) {
    if (c->dtype != CAAT_BF16 || T <= 64) return false;   // the MFMA tiles and K3's one pass
    if (!caat::psync_reads_final_private(c->P, c->h, c->dtype)) return false;
    const bool fused = fused_for(c, T);
    if (!fused && (long)c->P * T * c->h < PER_RANK_DIRECT_MIN) return false;
    const int first = fused ? c->n_s : (c->n_s + 7) / 8 * 8;
    return first < c->h;
}

// Row-parallel GEMM with the shared channels reduced over ranks inside the GEMM.
int run_row_reduce(const caat_ctx *c, int T, const void *in, const void *W2, void *S, void *Z,
                   hipStream_t s) {
    if (c->n_s > 0) {
        const int rc = run_gemm(c, shared_args(c, T, in, W2, S), s);
        if (rc != CAAT_OK) return rc;
    }
    if (c->n_s < c->h) return run_gemm(c, private_args(c, T, in, W2, Z), s);
    return CAAT_OK;
}

int run_gemm(const caat_ctx *c, const caat::GemmArgs &g, hipStream_t s) {
    if ((g.epi == caat::EPI_RESID || g.epi == caat::EPI_RESID_SPLIT) &&
        (c->dtype != CAAT_BF16 || caat::gemm_decode_applies(g)))
        return CAAT_EUNSUPPORTED;   // only the bf16 MFMA kernel has that epilogue
    if (c->dtype == CAAT_BF16) {
        if (!caat::gemm_bf16_supported(g)) return CAAT_EUNSUPPORTED;
        const hipError_t e = caat::gemm_decode_applies(g) ? caat::gemm_decode_bf16(g, s)
                                                          : caat::gemm_bf16(g, s);
        return e == hipSuccess ? CAAT_OK : CAAT_EDEVICE;
    }
    return caat::gemm_f32(g, s) == hipSuccess ? CAAT_OK : CAAT_EDEVICE;
}

int run_psync(const caat_ctx *c, int T, const void *partials, const void *resid,
              const void *gamma, const void *beta, void *out, void *out_resid, hipStream_t s,
              const void *S = nullptr, const void *priv_r = nullptr) {
    caat::PsyncArgs a{};
    a.S = S; a.s_ld = c->n_s; a.priv_r = priv_r;
    a.P = c->P; a.T = T; a.h = c->h; a.n_s = c->n_s; a.norm = c->norm;
    a.s_priv = c->s_priv; a.eps = c->eps;
    a.partials = partials; a.resid = resid; a.gamma = gamma;
    a.beta = (c->norm == CAAT_LAYERNORM) ? beta : nullptr;
    a.out = out; a.out_resid = out_resid;
    return caat::psync_norm(a, c->dtype, s) == hipSuccess ? CAAT_OK : CAAT_EDEVICE;
}

// T limit: every per-rank operand stays addressable with 32-bit byte offsets.
bool t_ok(const caat_ctx *c, int T) {
    if (T < 1) return false;
    const uint64_t widest = (uint64_t)(c->h > c->fs ? c->h : c->fs);
    return (uint64_t)T * widest * esize(c) < 0x80000000ull;
}

}  // namespace

CAAT_API int caat_create(caat_handle *out, int h, int ffn, int P, double p, int norm, int act,
                         int dtype) {
    if (out == nullptr) return CAAT_EINVAL;
    *out = nullptr;
    if (h < 8 || h > 16384 || h % 8 != 0) return CAAT_EINVAL;
    if (P < 1 || P > 16) return CAAT_EINVAL;
    if (!(p >= 0.0 && p <= 1.0)) return CAAT_EINVAL;  // also rejects NaN
    if (norm != CAAT_LAYERNORM && norm != CAAT_RMSNORM) return CAAT_EINVAL;
    if (act < CAAT_GELU || act > CAAT_NONE) return CAAT_EINVAL;
    if (dtype != CAAT_F32 && dtype != CAAT_BF16) return CAAT_EINVAL;
    int fs = 0, kin, k2;
    if (act == CAAT_NONE) {
        if (h % P != 0 || (h / P) % 8 != 0) return CAAT_EINVAL;
        kin = h / P;
        k2 = kin;
        ffn = 0;
    } else {
        if (ffn < P || ffn % P != 0 || (ffn / P) % 8 != 0) return CAAT_EINVAL;
        fs = ffn / P;
        kin = h;
        k2 = fs;
    }
    caat_ctx *c = new (std::nothrow) caat_ctx;
    if (c == nullptr) return CAAT_ENOMEM;
    memset(c, 0, sizeof(*c));
    c->h = h; c->ffn = ffn; c->P = P; c->fs = fs;
    c->F1 = (act == CAAT_SWIGLU) ? 2 * fs : fs;
    c->kin = kin; c->k2 = k2;
    c->n_s = shared_count(h, p);
    c->norm = norm; c->act = act; c->dtype = dtype;
    c->p = p; c->eps = 1e-5f; c->s_priv = 1.0f;
    *out = c;
    return CAAT_OK;
}

CAAT_API int caat_destroy(caat_handle handle) {
    delete handle;
    return CAAT_OK;
}

CAAT_API int caat_set_eps(caat_handle handle, float eps) {
    if (handle == nullptr || !(eps >= 0.0f) || isinf(eps)) return CAAT_EINVAL;
    handle->eps = eps;
    return CAAT_OK;
}

CAAT_API int caat_set_private_scale(caat_handle handle, float s) {
    if (handle == nullptr || !isfinite(s)) return CAAT_EINVAL;
    handle->s_priv = s;
    return CAAT_OK;
}

CAAT_API int caat_shared_channels(caat_handle handle) {
    return handle == nullptr ? CAAT_EINVAL : handle->n_s;
}

CAAT_API size_t caat_workspace_bytes(caat_handle handle, int T) {
    if (handle == nullptr || T < 1) return 0;
    return y_bytes(handle, T) + partial_bytes(handle, T) + s_bytes(handle, T);
}

CAAT_API int caat_set_workspace(caat_handle handle, void *dev_ptr, size_t bytes) {
    if (handle == nullptr) return CAAT_EINVAL;
    if (dev_ptr != nullptr && !aligned16(dev_ptr)) return CAAT_EINVAL;
    handle->ws = dev_ptr;
    handle->ws_bytes = dev_ptr ? bytes : 0;
    return CAAT_OK;
}

namespace {

std::mutex g_scratch_mu;
void *g_scratch[MAX_DEVICES];

int scratch_address(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return CAAT_EDEVICE;
    if (dev < 0 || dev >= MAX_DEVICES) return CAAT_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return CAAT_EDEVICE;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return CAAT_OK;
}

// The forward of one sublayer; preact (nullable, MLP only) also receives the raw
// pre-activation x W1^T, [P][T][F1].  events (nullable): hipEvent_t recorded on the
// stream after each step (CAAT_FWD_STEPS), for the caller's timing.
int scratch_address(void **out);

int forward_impl(caat_handle c, const caat_args *a, void *preact, void *const *events,
                 int n_events, bool static_ws = false) {
    if (c == nullptr || a == nullptr) return CAAT_EINVAL;
    const int T = a->T;
    if (T < 1) return CAAT_EINVAL;
    if (!aligned16(a->in) || !aligned16(a->W2) || !aligned16(a->gamma) || !aligned16(a->out))
        return CAAT_EINVAL;
    if (c->act != CAAT_NONE && !aligned16(a->W1)) return CAAT_EINVAL;
    if (!aligned16_or_null(a->resid) || !aligned16_or_null(a->beta) ||
        !aligned16_or_null(a->out_resid))
        return CAAT_EINVAL;
    if (n_events < 0 || (n_events > 0 && events == nullptr)) return CAAT_EINVAL;
    const void *resid = a->resid;
    if (resid == nullptr) {
        if (c->act == CAAT_NONE) return CAAT_EINVAL;  // H is [P][T][h/P]: not a residual
        resid = a->in;
    }
    if (!t_ok(c, T)) return CAAT_EUNSUPPORTED;
    const size_t need = caat_workspace_bytes(c, T);
    if (static_ws ? need > CAAT_SCRATCH_BYTES : (c->ws == nullptr || c->ws_bytes < need))
        return CAAT_EWORKSPACE;
    int rc = device_check();
    if (rc != CAAT_OK) return rc;
    void *wsp = c->ws;
    if (static_ws) {
        rc = scratch_address(&wsp);
        if (rc != CAAT_OK) return rc;
    }

    hipStream_t s = reinterpret_cast<hipStream_t>(a->stream);
    auto mark = [&](int k) -> int {
        if (k >= n_events || events[k] == nullptr) return CAAT_OK;
        return hipEventRecord(reinterpret_cast<hipEvent_t>(events[k]), s) == hipSuccess
                   ? CAAT_OK : CAAT_EDEVICE;
    };
#define CAAT_TRY(call) do { const int rc_ = (call); if (rc_ != CAAT_OK) return rc_; } while (0)
    char *ws = reinterpret_cast<char *>(wsp);
    void *Y = ws;
    void *Z = ws + y_bytes(c, T);
    void *S = ws + y_bytes(c, T) + partial_bytes(c, T);
    const void *gemm_in = a->in;
    // 0: the column-parallel GEMM and its activation (MLP only).
    if (c->act != CAAT_NONE) {
        caat::GemmArgs g = col_args(c, T, a->in, a->W1, Y);
        if (preact != nullptr) {
            if (c->dtype == CAAT_BF16 && !caat::gemm_decode_applies(g) &&
                !caat::gemm_bf16_rotates_k(g)) {
                // The MFMA kernel's epilogue stores the pre-activation beside Y (in the
                // K order of the backward's recompute GEMM).
                g.pre = preact; g.pre_stride = (size_t)T * c->F1; g.ld_pre = c->F1;
            } else {
                // Other kernels, and K orders rotated per tile: the backward's own
                // recompute GEMM, so that the two agree bit for bit.
                CAAT_TRY(run_gemm(c, preact_args(c, T, a->W1, a->in, preact), s));
            }
        }
        CAAT_TRY(run_gemm(c, g, s));
        gemm_in = Y;
    }
    CAAT_TRY(mark(0));
    if (fused_for(c, T)) {
        // 1, 2: the shared channels summed over ranks inside one GEMM, then the private
        // channels of every rank (bf16 with a residual output: added to the residual in
        // the GEMM's epilogue, straight into out_resid); 3: reduce-free K3 on S and the
        // private partials or rows.
        const bool priv_direct = a->out_resid != nullptr && private_direct_for(c, T);
        if (c->n_s > 0) CAAT_TRY(run_gemm(c, shared_args(c, T, gemm_in, a->W2, S), s));
        CAAT_TRY(mark(1));
        if (priv_direct)
            CAAT_TRY(run_gemm(c, private_resid_args(c, T, gemm_in, a->W2, resid, a->out_resid), s));
        else if (c->n_s < c->h)
            CAAT_TRY(run_gemm(c, private_args(c, T, gemm_in, a->W2, Z), s));
        CAAT_TRY(mark(2));
        CAAT_TRY(run_psync(c, T, Z, resid, a->gamma, a->beta, a->out, a->out_resid, s, S,
                           priv_direct ? a->out_resid : nullptr));
        return mark(3);
    }
    // 1: every rank's partials (bf16 with a residual output: the whole private chunks go
    // straight into out_resid with the residual added); 3: the partial channel-reduce,
    // residual and norm.
    const bool priv_direct = a->out_resid != nullptr && private_direct_for(c, T);
    CAAT_TRY(run_gemm(c, priv_direct ? row_resid_args(c, T, gemm_in, a->W2, Z, resid, a->out_resid)
                                     : row_args(c, T, gemm_in, a->W2, Z), s));
    CAAT_TRY(mark(1));
    CAAT_TRY(mark(2));
    CAAT_TRY(run_psync(c, T, Z, resid, a->gamma, a->beta, a->out, a->out_resid, s, nullptr,
                       priv_direct ? a->out_resid : nullptr));
    return mark(3);
#undef CAAT_TRY
}

}  // namespace

CAAT_API int caat_forward_ex(caat_handle c, const caat_args *a) {
    return forward_impl(c, a, nullptr, nullptr, 0);
}

CAAT_API int caat_forward_scratch(caat_handle c, const caat_args *a) {
    return forward_impl(c, a, nullptr, nullptr, 0, true);
}

CAAT_API int caat_forward_fused(caat_handle c, int T) {
    if (c == nullptr || T < 1) return CAAT_EINVAL;
    return fused_for(c, T) ? 1 : 0;
}

CAAT_API int caat_forward_private_in_epilogue(caat_handle c, int T) {
    if (c == nullptr || T < 1) return CAAT_EINVAL;
    return private_direct_for(c, T) ? 1 : 0;
}

CAAT_API int caat_forward_timed(caat_handle c, const caat_args *a, void *const *events,
                                int n_events) {
    return forward_impl(c, a, nullptr, events, n_events);
}

CAAT_API int caat_forward_train(caat_handle c, const caat_args *a, void *preact) {
    if (c == nullptr || c->act == CAAT_NONE || !aligned16(preact)) return CAAT_EINVAL;
    return forward_impl(c, a, preact, nullptr, 0);
}

CAAT_API int caat_forward(caat_handle c, int T, const void *x, const void *W1, const void *W2,
                          const void *gamma, void *out, void *stream) {
    if (c == nullptr) return CAAT_EINVAL;
    if (c->act == CAAT_NONE) return CAAT_EINVAL;
    caat_args a{};
    a.T = T; a.in = x; a.resid = x; a.W1 = W1; a.W2 = W2; a.gamma = gamma;
    a.beta = nullptr; a.out = out; a.out_resid = nullptr; a.stream = stream;
    return caat_forward_ex(c, &a);
}

CAAT_API int caat_column_gemm_act(caat_handle c, int T, const void *x, const void *W1, void *Y,
                                  void *stream) {
    if (c == nullptr || c->act == CAAT_NONE) return CAAT_EINVAL;
    if (T < 1 || !aligned16(x) || !aligned16(W1) || !aligned16(Y)) return CAAT_EINVAL;
    if (!t_ok(c, T)) return CAAT_EUNSUPPORTED;
    const int rc = device_check();
    if (rc != CAAT_OK) return rc;
    return run_gemm(c, col_args(c, T, x, W1, Y), reinterpret_cast<hipStream_t>(stream));
}

CAAT_API int caat_row_gemm(caat_handle c, int T, const void *in, const void *W2, void *partials,
                           void *stream) {
    if (c == nullptr) return CAAT_EINVAL;
    if (T < 1 || !aligned16(in) || !aligned16(W2) || !aligned16(partials)) return CAAT_EINVAL;
    if (!t_ok(c, T)) return CAAT_EUNSUPPORTED;
    const int rc = device_check();
    if (rc != CAAT_OK) return rc;
    return run_gemm(c, row_args(c, T, in, W2, partials), reinterpret_cast<hipStream_t>(stream));
}

CAAT_API int caat_row_gemm_reduce(caat_handle c, int T, const void *in, const void *W2, void *S,
                                  void *partials, void *stream) {
    if (c == nullptr) return CAAT_EINVAL;
    if (T < 1 || !aligned16(in) || !aligned16(W2)) return CAAT_EINVAL;
    if (c->n_s > 0 && !aligned16(S)) return CAAT_EINVAL;
    if (c->n_s < c->h && !aligned16(partials)) return CAAT_EINVAL;
    if (!fused_ok(c) || !t_ok(c, T)) return CAAT_EUNSUPPORTED;
    const int rc = device_check();
    if (rc != CAAT_OK) return rc;
    return run_row_reduce(c, T, in, W2, S, partials, reinterpret_cast<hipStream_t>(stream));
}

CAAT_API int caat_sync_norm(caat_handle c, int T, const void *S, const void *partials,
                            const void *resid, const void *gamma, const void *beta, void *out,
                            void *out_resid, void *stream) {
    if (c == nullptr || T < 1) return CAAT_EINVAL;
    if (c->n_s > 0 && !aligned16(S)) return CAAT_EINVAL;
    if (c->n_s < c->h && !aligned16(partials)) return CAAT_EINVAL;
    if (!aligned16(resid) || !aligned16(gamma) || !aligned16(out)) return CAAT_EINVAL;
    if (!aligned16_or_null(beta) || !aligned16_or_null(out_resid)) return CAAT_EINVAL;
    if (!fused_ok(c) || !t_ok(c, T)) return CAAT_EUNSUPPORTED;
    const int rc = device_check();
    if (rc != CAAT_OK) return rc;
    // With n_s == h no private column is read; any aligned pointer stands in.
    const void *Z = (c->n_s < c->h) ? partials : resid;
    const void *Sv = (c->n_s > 0) ? S : resid;
    return run_psync(c, T, Z, resid, gamma, beta, out, out_resid,
                     reinterpret_cast<hipStream_t>(stream), Sv);
}

CAAT_API int caat_partial_sync_norm(caat_handle c, int T, const void *partials, const void *resid,
                                    const void *gamma, const void *beta, void *out,
                                    void *out_resid, void *stream) {
    if (c == nullptr || T < 1) return CAAT_EINVAL;
    if (!aligned16(partials) || !aligned16(resid) || !aligned16(gamma) || !aligned16(out))
        return CAAT_EINVAL;
    if (!aligned16_or_null(beta) || !aligned16_or_null(out_resid)) return CAAT_EINVAL;
    if (!t_ok(c, T)) return CAAT_EUNSUPPORTED;
    const int rc = device_check();
    if (rc != CAAT_OK) return rc;
    return run_psync(c, T, partials, resid, gamma, beta, out, out_resid,
                     reinterpret_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------------
// Backward (§4 "Forward-backward mismatch", Eq. 10-13; App. B, Eq. 26-30).

namespace {

size_t round8(size_t n) { return (n + 7) & ~(size_t)7; }

// Workspace of the backward, in this order (each part 256-byte aligned).  Tp = T
// rounded up to a multiple of 8: the transposed activations are the operands of the
// weight-gradient GEMMs, whose contraction runs over tokens.
struct BwdLayout {
    size_t dzt, dres, gpart, bpart, W2T, dY, dztT, YT, A, da, Y, W1T, xT, daT, total;
};

// bf16 weight gradients contract over tokens straight from the token-major operands
// (gemm_tn); otherwise (fp32, or widths not a multiple of 8) through transposed copies.
bool tn_weight_grads(const caat_ctx *c) {
    return c->dtype == CAAT_BF16 && c->h % 8 == 0 && c->k2 % 8 == 0 && c->F1 % 8 == 0;
}

BwdLayout bwd_layout(const caat_ctx *c, int T) {
    BwdLayout L{};
    const size_t E = esize(c), P = c->P, h = c->h, k2 = c->k2, F1 = c->F1, fs = c->fs;
    const size_t Tp = round8(T), NB = caat::psync_bwd_blocks(T);
    const bool tr = !tn_weight_grads(c);
    size_t off = 0;
    auto take = [&](size_t n) { const size_t o = off; off += align256(n); return o; };
    L.dzt = take(P * T * h * E);
    L.dres = take(P * T * h * E);
    L.gpart = take(NB * h * 4);
    L.bpart = take(NB * h * 4);
    L.W2T = take(P * k2 * h * E);
    L.dY = take(P * T * k2 * E);
    if (tr) {
        L.dztT = take(P * h * Tp * E);
        L.YT = take(P * k2 * Tp * E);
    }
    if (c->act != CAAT_NONE) {
        L.A = take(P * T * F1 * E);
        L.da = take(P * T * F1 * E);
        L.Y = take(P * T * fs * E);
        L.W1T = take(P * h * F1 * E);
        if (tr) {
            L.xT = take(P * h * Tp * E);
            L.daT = take(P * F1 * Tp * E);
        }
    }
    L.total = off;
    return L;
}

// Weight gradient out[m][n] = sum_t A[t][m] B[t][n] per rank, from token-major A [T][M]
// and B [T][N] (gemm_tn).
int run_tn(const caat_ctx *c, int T, int M, int N, const void *A, const void *B, void *out,
           hipStream_t s) {
    caat::TnArgs t{};
    t.P = c->P; t.M = M; t.N = N; t.K = T;
    t.A = A; t.a_stride = (size_t)T * M; t.lda = M;
    t.B = B; t.b_stride = (size_t)T * N; t.ldb = N;
    t.out = out; t.o_stride = (size_t)M * N; t.ldo = N;
    if (!caat::gemm_tn_supported(t)) return CAAT_EUNSUPPORTED;
    return caat::gemm_tn_bf16(t, s) == hipSuccess ? CAAT_OK : CAAT_EDEVICE;
}

// B3's share of the workspace (the per-workgroup norm-parameter partials).
size_t bwd_norm_bytes(const caat_ctx *c, int T) {
    return 2 * align256((size_t)caat::psync_bwd_blocks(T) * c->h * 4);
}

bool t_ok_bwd(const caat_ctx *c, int T) {
    if (!t_ok(c, T)) return false;
    const uint64_t widest = (uint64_t)(c->h > c->F1 ? c->h : c->F1);
    return (uint64_t)round8(T) * widest * esize(c) < 0x80000000ull;
}

// One plain NT GEMM: out[m][t][n] = sum_k W[m][n][k] X[m][t][k], row stride ldo = N.
caat::GemmArgs plain_args(const caat_ctx *c, int rows, int N, int K, const void *W,
                          const void *X, void *out) {
    caat::GemmArgs g{};
    g.P = c->P; g.N = N; g.T = rows; g.K = K;
    g.W = W; g.w_stride = (size_t)N * K;
    g.X = X; g.x_stride = (size_t)rows * K;
    g.out = out; g.o_stride = (size_t)rows * N; g.ldo = N;
    g.up_off = 0;
    g.epi = caat::EPI_STORE;
    g.kseg = 1;
    return g;
}

int run_psync_bwd(const caat_ctx *c, int T, const void *r, const void *dout, const void *dres,
                  const void *gamma, void *dzt, void *dresid, float *dgamma, float *dbeta,
                  char *ws, hipStream_t s) {
    caat::PsyncBwdArgs b{};
    b.P = c->P; b.T = T; b.h = c->h; b.n_s = c->n_s; b.norm = c->norm;
    b.s_priv = c->s_priv; b.eps = c->eps;
    b.r = r; b.dout = dout; b.dres = dres; b.gamma = gamma;
    b.dzt = dzt; b.dresid = dresid;
    b.nblk = caat::psync_bwd_blocks(T);
    b.gpart = reinterpret_cast<float *>(ws);
    b.bpart = reinterpret_cast<float *>(ws + bwd_norm_bytes(c, T) / 2);
    if (caat::psync_norm_bwd(b, c->dtype, s) != hipSuccess) return CAAT_EDEVICE;
    if (caat::colsum_f32(b.gpart, b.nblk, c->h, dgamma, s) != hipSuccess) return CAAT_EDEVICE;
    if (dbeta != nullptr) {
        // RMSNorm has no beta: its gradient is written as zero (a sum over no rows).
        const int rows = (c->norm == CAAT_LAYERNORM) ? b.nblk : 0;
        if (caat::colsum_f32(b.bpart, rows, c->h, dbeta, s) != hipSuccess) return CAAT_EDEVICE;
    }
    return CAAT_OK;
}

}  // namespace

CAAT_API size_t caat_backward_workspace_bytes(caat_handle handle, int T) {
    if (handle == nullptr || T < 1) return 0;
    return bwd_layout(handle, T).total;
}

CAAT_API int caat_partial_sync_norm_backward(caat_handle c, int T, const void *out_resid,
                                             const void *dout, const void *dres,
                                             const void *gamma, void *dpartials, void *dresid,
                                             float *dgamma, float *dbeta, void *workspace,
                                             size_t workspace_bytes, void *stream) {
    if (c == nullptr || T < 1) return CAAT_EINVAL;
    if (!aligned16(out_resid) || !aligned16(dout) || !aligned16(gamma) || !aligned16(dpartials) ||
        !aligned16(dgamma))
        return CAAT_EINVAL;
    if (!aligned16_or_null(dres) || !aligned16_or_null(dresid) || !aligned16_or_null(dbeta))
        return CAAT_EINVAL;
    if (!t_ok(c, T)) return CAAT_EUNSUPPORTED;
    if (!aligned16(workspace) || workspace_bytes < bwd_norm_bytes(c, T)) return CAAT_EWORKSPACE;
    const int rc = device_check();
    if (rc != CAAT_OK) return rc;
    return run_psync_bwd(c, T, out_resid, dout, dres, gamma, dpartials, dresid, dgamma, dbeta,
                         reinterpret_cast<char *>(workspace), reinterpret_cast<hipStream_t>(stream));
}

CAAT_API int caat_backward(caat_handle c, const caat_bwd_args *a) {
    if (c == nullptr || a == nullptr) return CAAT_EINVAL;
    const int T = a->T;
    if (T < 1) return CAAT_EINVAL;
    const bool mlp = c->act != CAAT_NONE;
    if (!aligned16(a->in) || !aligned16(a->W2) || !aligned16(a->gamma) ||
        !aligned16(a->out_resid) || !aligned16(a->dout) || !aligned16(a->din) ||
        !aligned16(a->dW2) || !aligned16(a->dgamma))
        return CAAT_EINVAL;
    if (mlp && (!aligned16(a->W1) || !aligned16(a->dW1))) return CAAT_EINVAL;
    if (!aligned16_or_null(a->preact) || (!mlp && a->preact != nullptr)) return CAAT_EINVAL;
    if (!aligned16_or_null(a->dres) || !aligned16_or_null(a->dresid) ||
        !aligned16_or_null(a->dbeta))
        return CAAT_EINVAL;
    if (a->dresid == nullptr && !mlp) return CAAT_EINVAL;  // H is not a residual
    if (!t_ok_bwd(c, T)) return CAAT_EUNSUPPORTED;
    const BwdLayout L = bwd_layout(c, T);
    if (!aligned16(a->workspace) || a->workspace_bytes < L.total) return CAAT_EWORKSPACE;
    int rc = device_check();
    if (rc != CAAT_OK) return rc;

    hipStream_t s = reinterpret_cast<hipStream_t>(a->stream);
    char *ws = reinterpret_cast<char *>(a->workspace);
    const int P = c->P, h = c->h, k2 = c->k2, F1 = c->F1, fs = c->fs, Tp = (int)round8(T);
    const bool tn = tn_weight_grads(c);
    void *dzt = ws + L.dzt;
    void *dresid = a->dresid ? a->dresid : ws + L.dres;
#define CAAT_TRY(call) do { const int rc_ = (call); if (rc_ != CAAT_OK) return rc_; } while (0)
#define CAAT_HIP(call) do { if ((call) != hipSuccess) return CAAT_EDEVICE; } while (0)
    int step = 0;
    auto mark = [&]() -> int {   // the caller's timing event after each step
        if (a->events != nullptr && step < a->n_events &&
            hipEventRecord(reinterpret_cast<hipEvent_t>(a->events[step]), s) != hipSuccess)
            return CAAT_EDEVICE;
        ++step;
        return CAAT_OK;
    };
    // 0: norm derivative per rank, then the reduce over ranks of the shared channels.
    CAAT_TRY(run_psync_bwd(c, T, a->out_resid, a->dout, a->dres, a->gamma, dzt, dresid,
                           a->dgamma, a->dbeta, ws + L.gpart, s));
    CAAT_TRY(mark());
    // 1, 2: second GEMM, dY = dZt W2 (per rank), through W2^T [k2][h].
    CAAT_HIP(caat::transpose(a->W2, ws + L.W2T, P, h, k2, h, c->dtype, s));
    CAAT_TRY(mark());
    void *dY = mlp ? ws + L.dY : a->din;   // out-projection: dY is dH
    CAAT_TRY(run_gemm(c, plain_args(c, T, k2, h, ws + L.W2T, dzt, dY), s));
    CAAT_TRY(mark());
    const void *y_in = a->in;              // the second GEMM's input (H for the out-projection)
    if (mlp) {
        // 3, 4: the pre-activation (stored by caat_forward_train, or recomputed), then
        // da = dY * sigma'(a) and Y = sigma(a).
        const void *pre = a->preact;
        if (pre == nullptr) {
            CAAT_TRY(run_gemm(c, preact_args(c, T, a->W1, a->in, ws + L.A), s));
            pre = ws + L.A;
        }
        CAAT_TRY(mark());
        CAAT_HIP(caat::act_backward(c->act, c->dtype, (size_t)P * T, fs, pre, dY, ws + L.da,
                                    ws + L.Y, s));
        CAAT_TRY(mark());
        y_in = ws + L.Y;
        // 5, 6: first GEMM, dx = da W1, through W1^T [h][F1].
        CAAT_HIP(caat::transpose(a->W1, ws + L.W1T, P, F1, h, F1, c->dtype, s));
        CAAT_TRY(mark());
        CAAT_TRY(run_gemm(c, plain_args(c, T, h, F1, ws + L.W1T, ws + L.da, a->din), s));
        if (a->dresid == nullptr)
            CAAT_HIP(caat::add_inplace(a->din, dresid, (size_t)P * T * h, c->dtype, s));
        CAAT_TRY(mark());
        // 7, 8: dW1 = da^T x: contraction over tokens (bf16: from the token-major
        // operands; else through transposed copies).
        if (tn) {
            CAAT_TRY(mark());
            CAAT_TRY(run_tn(c, T, F1, h, ws + L.da, a->in, a->dW1, s));
        } else {
            CAAT_HIP(caat::transpose(ws + L.da, ws + L.daT, P, T, F1, Tp, c->dtype, s));
            CAAT_HIP(caat::transpose(a->in, ws + L.xT, P, T, h, Tp, c->dtype, s));
            CAAT_TRY(mark());
            CAAT_TRY(run_gemm(c, plain_args(c, F1, h, Tp, ws + L.xT, ws + L.daT, a->dW1), s));
        }
        CAAT_TRY(mark());
    } else {
        for (int k = 3; k <= 8; ++k) CAAT_TRY(mark());
    }
    // 9, 10: dW2 = dZt^T Y (or dZt^T H): contraction over tokens.
    if (tn) {
        CAAT_TRY(mark());
        CAAT_TRY(run_tn(c, T, h, k2, dzt, y_in, a->dW2, s));
    } else {
        CAAT_HIP(caat::transpose(y_in, ws + L.YT, P, T, k2, Tp, c->dtype, s));
        CAAT_HIP(caat::transpose(dzt, ws + L.dztT, P, T, h, Tp, c->dtype, s));
        CAAT_TRY(mark());
        CAAT_TRY(run_gemm(c, plain_args(c, h, k2, Tp, ws + L.YT, ws + L.dztT, a->dW2), s));
    }
    CAAT_TRY(mark());
#undef CAAT_TRY
#undef CAAT_HIP
    return CAAT_OK;
}

// ---------------------------------------------------------------------------------
// The full block with logical devices: QKV projection, attention core, the out-projection
// sublayer and the MLP sublayer (App. A Eq. 16 / 18 / 24, Eq. 22; §3.2; §4 Eq. 9).

namespace {

bool attn_shape_ok(int P, int T, int S, int nh, int d) {
    if (P < 1 || P > 16 || T < 1 || S < 1 || nh < 1 || (d != 64 && d != 128)) return false;
    if (T % S != 0 || S % 8 != 0) return false;
    // 32-bit byte offsets inside one rank's QKV rows and V^T rows.
    return (uint64_t)T * 3 * nh * d * 2 < 0x80000000ull &&
           (uint64_t)d * round8(T) * 2 < 0x80000000ull;
}

size_t attn_ws_bytes(int P, int T, int nh, int d) {
    return align256((size_t)P * nh * d * round8(T) * 2);
}

int run_attention(int P, int T, int S, int nh, int d, const void *qkv, void *H, void *vt,
                  hipStream_t s, void *mid_event = nullptr) {
    const int hp = nh * d, Tp = (int)round8(T);
    // V^T [P][nh d][Tp] from the V columns of qkv (rows 3 hp apart).
    if (caat::transpose_strided(reinterpret_cast<const char *>(qkv) + (size_t)2 * hp * 2, vt, P, T,
                                hp, Tp, 3 * hp, (size_t)T * 3 * hp, CAAT_BF16, s) != hipSuccess)
        return CAAT_EDEVICE;
    if (mid_event != nullptr &&
        hipEventRecord(reinterpret_cast<hipEvent_t>(mid_event), s) != hipSuccess)
        return CAAT_EDEVICE;
    caat::AttnArgs a{};
    a.P = P; a.T = T; a.S = S; a.nh = nh; a.d = d;
    a.qkv = qkv; a.vt = vt; a.Tp = Tp; a.H = H;
    return caat::attention_bf16(a, s) == hipSuccess ? CAAT_OK : CAAT_EDEVICE;
}

struct BlockLayout { size_t qkv, vt, H, a_out, a_res, total; };

BlockLayout block_layout(const caat_ctx *attn, int nh, int T) {
    BlockLayout L{};
    const size_t P = attn->P, h = attn->h, hp = h / P, d = hp / nh;
    size_t off = 0;
    auto take = [&](size_t n) { const size_t o = off; off += align256(n); return o; };
    L.qkv = take(P * T * 3 * hp * 2);
    L.vt = take(attn_ws_bytes((int)P, T, nh, (int)d));
    L.H = take(P * T * hp * 2);
    L.a_out = take(P * T * h * 2);
    L.a_res = take(P * T * h * 2);
    L.total = off;
    return L;
}

int block_check(const caat_ctx *attn, const caat_ctx *mlp, int nh) {
    if (attn == nullptr || mlp == nullptr) return CAAT_EINVAL;
    if (attn->act != CAAT_NONE || mlp->act == CAAT_NONE) return CAAT_EINVAL;
    if (attn->h != mlp->h || attn->P != mlp->P || attn->norm != mlp->norm) return CAAT_EINVAL;
    if (attn->dtype != CAAT_BF16 || mlp->dtype != CAAT_BF16) return CAAT_EUNSUPPORTED;
    if (nh < 1 || attn->kin % nh != 0) return CAAT_EINVAL;
    const int d = attn->kin / nh;
    if (d != 64 && d != 128) return CAAT_EUNSUPPORTED;
    return CAAT_OK;
}

}  // namespace

CAAT_API size_t caat_attention_workspace_bytes(int P, int T, int nh, int d) {
    if (P < 1 || T < 1 || nh < 1 || d < 1) return 0;
    return attn_ws_bytes(P, T, nh, d);
}

CAAT_API int caat_attention(int P, int T, int S, int nh, int d, const void *qkv, void *H,
                            void *workspace, size_t workspace_bytes, void *stream) {
    if (!aligned16(qkv) || !aligned16(H)) return CAAT_EINVAL;
    if (P < 1 || T < 1 || S < 1 || nh < 1) return CAAT_EINVAL;
    if (T % S != 0 || S % 8 != 0) return CAAT_EINVAL;
    if (!attn_shape_ok(P, T, S, nh, d)) return CAAT_EUNSUPPORTED;
    if (!aligned16(workspace) || workspace_bytes < attn_ws_bytes(P, T, nh, d))
        return CAAT_EWORKSPACE;
    const int rc = device_check();
    if (rc != CAAT_OK) return rc;
    return run_attention(P, T, S, nh, d, qkv, H, workspace, reinterpret_cast<hipStream_t>(stream));
}

CAAT_API size_t caat_block_workspace_bytes(caat_handle attn, caat_handle mlp, int nh, int T) {
    if (T < 1 || block_check(attn, mlp, nh) != CAAT_OK) return 0;
    return block_layout(attn, nh, T).total;
}

CAAT_API int caat_block_forward(caat_handle attn, caat_handle mlp, int nh, const caat_block_args *a) {
    if (a == nullptr) return CAAT_EINVAL;
    int rc = block_check(attn, mlp, nh);
    if (rc != CAAT_OK) return rc;
    const int T = a->T, S = a->S, P = attn->P, h = attn->h, hp = attn->kin, d = hp / nh;
    if (T < 1 || S < 1 || T % S != 0 || S % 8 != 0) return CAAT_EINVAL;
    if (!aligned16(a->in) || !aligned16(a->resid) || !aligned16(a->Wqkv) || !aligned16(a->Wo) ||
        !aligned16(a->W1) || !aligned16(a->W2) || !aligned16(a->gamma_attn) ||
        !aligned16(a->gamma_mlp) || !aligned16(a->out) || !aligned16(a->out_resid))
        return CAAT_EINVAL;
    if (!aligned16_or_null(a->beta_attn) || !aligned16_or_null(a->beta_mlp)) return CAAT_EINVAL;
    if (!attn_shape_ok(P, T, S, nh, d) || !t_ok(attn, T) || !t_ok(mlp, T)) return CAAT_EUNSUPPORTED;
    const BlockLayout L = block_layout(attn, nh, T);
    if (!aligned16(a->workspace) || a->workspace_bytes < L.total) return CAAT_EWORKSPACE;
    if (attn->ws == nullptr || attn->ws_bytes < caat_workspace_bytes(attn, T) ||
        mlp->ws == nullptr || mlp->ws_bytes < caat_workspace_bytes(mlp, T))
        return CAAT_EWORKSPACE;
    rc = device_check();
    if (rc != CAAT_OK) return rc;

    hipStream_t s = reinterpret_cast<hipStream_t>(a->stream);
    char *ws = reinterpret_cast<char *>(a->workspace);
    // QKV projection per rank (column-parallel: the rank's heads), then attention.
    caat::GemmArgs g{};
    g.P = P; g.N = 3 * hp; g.T = T; g.K = h;
    g.W = a->Wqkv; g.w_stride = (size_t)3 * hp * h;
    g.X = a->in; g.x_stride = (size_t)T * h;
    g.out = ws + L.qkv; g.o_stride = (size_t)T * 3 * hp; g.ldo = 3 * hp;
    g.epi = caat::EPI_STORE; g.kseg = 1;
    auto ev = [&](int k) -> void * {
        return (a->events != nullptr && k < a->n_events) ? a->events[k] : nullptr;
    };
    auto mark = [&](int k) -> int {
        return (ev(k) == nullptr ||
                hipEventRecord(reinterpret_cast<hipEvent_t>(ev(k)), s) == hipSuccess)
                   ? CAAT_OK : CAAT_EDEVICE;
    };
    rc = run_gemm(attn, g, s);
    if (rc == CAAT_OK) rc = mark(0);
    if (rc != CAAT_OK) return rc;
    rc = run_attention(P, T, S, nh, d, ws + L.qkv, ws + L.H, ws + L.vt, s, ev(1));
    if (rc == CAAT_OK) rc = mark(2);
    if (rc != CAAT_OK) return rc;
    // The two sublayers, through the handles' own workspaces.
    caat_args sa{};
    sa.T = T; sa.in = ws + L.H; sa.resid = a->resid; sa.W1 = nullptr; sa.W2 = a->Wo;
    sa.gamma = a->gamma_attn; sa.beta = a->beta_attn; sa.out = ws + L.a_out;
    sa.out_resid = ws + L.a_res; sa.stream = a->stream;
    rc = caat_forward_ex(attn, &sa);
    if (rc == CAAT_OK) rc = mark(3);
    if (rc != CAAT_OK) return rc;
    caat_args sm{};
    sm.T = T; sm.in = ws + L.a_out; sm.resid = ws + L.a_res; sm.W1 = a->W1; sm.W2 = a->W2;
    sm.gamma = a->gamma_mlp; sm.beta = a->beta_mlp; sm.out = a->out; sm.out_resid = a->out_resid;
    sm.stream = a->stream;
    rc = caat_forward_ex(mlp, &sm);
    if (rc == CAAT_OK) rc = mark(4);
    return rc;
}

CAAT_API const char *caat_error_string(int code) {
    switch (code) {
    case CAAT_OK: return "success";
    case CAAT_EINVAL: return "invalid argument";
    case CAAT_ENOMEM: return "host allocation failed";
    case CAAT_EWORKSPACE: return "workspace missing or too small";
    case CAAT_EDEVICE: return "HIP call or kernel launch failed";
    case CAAT_EUNSUPPORTED: return "unsupported device or size";
    default: return "unknown status";
    }
}
