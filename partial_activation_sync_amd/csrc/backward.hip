// Backward of the CAAT sublayer: the kernels that are not GEMMs.
//
// "Tensor-Parallelism with Partially Synchronized Activations", §4 "Forward-backward
// mismatch" (Eq. 9-13) and App. B (Eq. 25-30).  With partially synchronized
// activations the ranks' norm derivatives differ, so the reduce over ranks of the
// backward must come after the norm derivative (the 'h' placement), and the norm
// parameters' gradients are summed over ranks.  §4 also asks for the reduced
// gradients to be accumulated in 32-bit: here the sum over ranks runs in fp32
// registers on the fp32 values of g (no 16-bit payload exists on one device).
//
// B3 (k_psync_norm_bwd), per token t and rank m, r = out_resid of the forward:
//   nhat = (r - mean) * inv,  dnhat = dout * gamma,
//   g_m  = inv * (dnhat - nhat * mean(dnhat * nhat) [- mean(dnhat) for LayerNorm]) + dres
//   dZt_m[l] = sum_q g_q[l] (l < n_s, fp32, ranks ascending),  s_priv * g_m[l] otherwise
//   dresid_m = g_m;  dgamma += dout * nhat,  dbeta += dout   (per workgroup, fp32)
// One workgroup loops over tokens t = blockIdx.x, blockIdx.x + gridDim.x, ...; thread
// i owns the 8-channel chunks i + j * blockDim of every rank, so the per-channel
// parameter gradients stay in registers across tokens and are written once per
// workgroup, then summed over workgroups in a fixed order (colsum_f32): deterministic.
#include "caat_internal.h"
#include "rowops.h"

namespace caat {
namespace {

// Workgroups of the norm backward: one per CU is what its registers allow, and each
// adds one row of norm-parameter partials.
constexpr int BWD_MAX_BLOCKS = 256;
constexpr int BWD_MAX_WAVES = 8;

template <int NCH, int GB, int NORM, typename TIO>
__global__ __launch_bounds__(512) void k_psync_norm_bwd(PsyncBwdArgs a)
{
    // Two reduction buffers used in turn, so consecutive block sums need one barrier each.
    __shared__ float red[2][BWD_MAX_WAVES * 2 * GB];
    const int P = a.P, T = a.T, h = a.h, n_s = a.n_s;
    const size_t rs = (size_t)T * h;
    const TIO *Rv = reinterpret_cast<const TIO *>(a.r);
    const TIO *Dv = reinterpret_cast<const TIO *>(a.dout);
    const TIO *DRv = reinterpret_cast<const TIO *>(a.dres);
    TIO *DZ = reinterpret_cast<TIO *>(a.dzt);
    TIO *DRES = reinterpret_cast<TIO *>(a.dresid);
    const int nchunk = h / 8;
    const float inv_h = 1.0f / (float)h;

    int c[NCH];
    bool ok[NCH];
    float gam[NCH][8], gacc[NCH][8], bacc[NCH][8];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        c[j] = threadIdx.x + j * blockDim.x;
        ok[j] = c[j] < nchunk;
        if (ok[j]) {
            Vec8<TIO>::load(reinterpret_cast<const TIO *>(a.gamma) + c[j] * 8, gam[j]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) gam[j][e] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) gacc[j][e] = bacc[j][e] = 0.f;
    }

    // The (token, rank group) pairs of this workgroup in order; where the registers allow,
    // software-pipelined: the loads of the next pair are in flight while the current one
    // is reduced and stored.
    const int ngroups = (P + GB - 1) / GB;
    const int ntok = (int)blockIdx.x < T ? (T - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
    const int niter = ntok * ngroups;
    float sg[NCH][8];
    // Every load of a pair at once, kept in the storage format (zero past the end).
    auto issue = [&](int it, Raw<TIO> (&rr)[GB][NCH], Raw<TIO> (&dd)[GB][NCH],
                     Raw<TIO> (&ee)[GB][NCH]) {
        const bool live = it < niter;
        const int t = blockIdx.x + (it / ngroups) * gridDim.x, g0 = (it % ngroups) * GB;
        const size_t row = (size_t)t * h;
#pragma unroll
        for (int q = 0; q < GB; ++q) {
            const int m = g0 + q;
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                if (live && m < P && ok[j]) {
                    const size_t off = m * rs + row + c[j] * 8;
                    rr[q][j].load(Rv + off);
                    dd[q][j].load(Dv + off);
                    if (DRv) ee[q][j].load(DRv + off); else ee[q][j].zero();
                } else {
                    rr[q][j].zero();
                    dd[q][j].zero();
                    ee[q][j].zero();
                }
            }
        }
    };
    auto process = [&](int it, Raw<TIO> (&rr)[GB][NCH], Raw<TIO> (&dd)[GB][NCH],
                       Raw<TIO> (&ee)[GB][NCH]) {
        const int t = blockIdx.x + (it / ngroups) * gridDim.x, g0 = (it % ngroups) * GB;
        const size_t row = (size_t)t * h;
        if (g0 == 0) {
#pragma unroll
            for (int j = 0; j < NCH; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e) sg[j][e] = 0.f;
        }
        {
            // Row statistics of r (fp32), as the forward normalization computes them.
            float mean[GB], inv[GB];
            {
                float s[GB];
#pragma unroll
                for (int q = 0; q < GB; ++q) {
                    float acc = 0.f;
#pragma unroll
                    for (int j = 0; j < NCH; ++j) {
                        float v[8];
                        rr[q][j].unpack(v);
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc += v[e];
                    }
                    s[q] = acc;
                }
                if (NORM == CAAT_LAYERNORM) {
                    block_sum<GB>(s, red[0]);
#pragma unroll
                    for (int q = 0; q < GB; ++q) mean[q] = s[q] * inv_h;
                } else {
#pragma unroll
                    for (int q = 0; q < GB; ++q) mean[q] = 0.f;
                }
            }
            {
                float s[GB];
#pragma unroll
                for (int q = 0; q < GB; ++q) {
                    float acc = 0.f;
#pragma unroll
                    for (int j = 0; j < NCH; ++j) {
                        float v[8];
                        rr[q][j].unpack(v);
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float d = ok[j] ? v[e] - mean[q] : 0.f;
                            acc += d * d;
                        }
                    }
                    s[q] = acc;
                }
                block_sum<GB>(s, red[1]);
#pragma unroll
                for (int q = 0; q < GB; ++q) inv[q] = rsqrtf(s[q] * inv_h + a.eps);
            }
            // mean(dnhat) and mean(dnhat * nhat) of every rank of the group.
            float s12[2 * GB];
#pragma unroll
            for (int q = 0; q < GB; ++q) {
                float s1 = 0.f, s2 = 0.f;
#pragma unroll
                for (int j = 0; j < NCH; ++j) {
                    float v[8], d[8];
                    rr[q][j].unpack(v);
                    dd[q][j].unpack(d);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float dn = d[e] * gam[j][e];
                        const float nh = ok[j] ? (v[e] - mean[q]) * inv[q] : 0.f;
                        s1 += dn;
                        s2 += dn * nh;
                    }
                }
                s12[q] = s1;
                s12[GB + q] = s2;
            }
            block_sum<2 * GB>(s12, red[0]);

#pragma unroll
            for (int q = 0; q < GB; ++q) {
                const int m = g0 + q;
                if (m >= P) break;
                const float s1 = (NORM == CAAT_LAYERNORM) ? s12[q] * inv_h : 0.f;
                const float s2 = s12[GB + q] * inv_h;
#pragma unroll
                for (int j = 0; j < NCH; ++j) {
                    if (!ok[j]) continue;
                    const int l0 = c[j] * 8;
                    const size_t off = m * rs + row + l0;
                    float v[8], d[8], dr[8], gv[8];
                    rr[q][j].unpack(v);
                    dd[q][j].unpack(d);
                    ee[q][j].unpack(dr);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float nh = (v[e] - mean[q]) * inv[q];
                        const float dn = d[e] * gam[j][e];
                        gv[e] = inv[q] * (dn - nh * s2 - s1) + dr[e];
                        gacc[j][e] += d[e] * nh;
                        bacc[j][e] += d[e];
                    }
                    if (DRES) Vec8<TIO>::store(DRES + off, gv);
                    if (l0 + 8 <= n_s) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) sg[j][e] += gv[e];
                    } else if (l0 >= n_s) {
                        float pv[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) pv[e] = a.s_priv * gv[e];
                        Vec8<TIO>::store(DZ + off, pv);
                    } else {
                        // The chunk that holds the shared/private boundary.
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            if (l0 + e < n_s) sg[j][e] += gv[e];
                            else DZ[off + e] = static_cast<TIO>(a.s_priv * gv[e]);
                        }
                    }
                }
            }
            // red[0] is written again by the next pair's first block sum.
            __syncthreads();
        }
        if (g0 + GB >= P) {
            // Shared channels: every rank's partial receives the sum over ranks.
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                if (!ok[j]) continue;
                const int l0 = c[j] * 8;
                if (l0 >= n_s) continue;
                for (int m = 0; m < P; ++m) {
                    const size_t off = m * rs + row + l0;
                    if (l0 + 8 <= n_s) {
                        Vec8<TIO>::store(DZ + off, sg[j]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (l0 + e < n_s) DZ[off + e] = static_cast<TIO>(sg[j][e]);
                    }
                }
            }
        }
    };
    Raw<TIO> rA[GB][NCH], dA[GB][NCH], eA[GB][NCH];
    if constexpr (NCH == 1 && sizeof(TIO) == 2) {
        // Two register sets in turn (the wider shapes and fp32 have no room for them).
        Raw<TIO> rB[GB][NCH], dB[GB][NCH], eB[GB][NCH];
        issue(0, rA, dA, eA);
        for (int it = 0; it < niter; it += 2) {
            issue(it + 1, rB, dB, eB);
            process(it, rA, dA, eA);
            issue(it + 2, rA, dA, eA);
            if (it + 1 < niter) process(it + 1, rB, dB, eB);
        }
    } else {
        for (int it = 0; it < niter; ++it) {
            issue(it, rA, dA, eA);
            process(it, rA, dA, eA);
        }
    }

#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        if (!ok[j]) continue;
        const size_t off = (size_t)blockIdx.x * h + c[j] * 8;
        Vec8<float>::store(a.gpart + off, gacc[j]);
        Vec8<float>::store(a.bpart + off, bacc[j]);
    }
}

template <int NORM, typename TIO>
hipError_t launch_bwd(const PsyncBwdArgs &a, hipStream_t s) {
    const int chunks = a.h / 8;
    const int nch = chunks <= 512 ? 1 : chunks <= 1024 ? 2 : 4;
    int threads = (chunks + nch - 1) / nch;
    threads = ((threads + 63) / 64) * 64;
    const dim3 grid(a.nblk), block(threads);
    switch (nch) {
    case 1: hipLaunchKernelGGL((k_psync_norm_bwd<1, 4, NORM, TIO>), grid, block, 0, s, a); break;
    // Fewer ranks per group as the chunks per thread grow, so the raw rows of a group
    // stay in registers.
    case 2: hipLaunchKernelGGL((k_psync_norm_bwd<2, 2, NORM, TIO>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((k_psync_norm_bwd<4, 1, NORM, TIO>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

// 64 columns per workgroup; the 4 waves take rows r = wave (mod 4), each lane summing
// its column in ascending row order, then the 4 partial sums are added in wave order.
__global__ __launch_bounds__(256) void k_colsum(const float *__restrict__ part, int rows, int h,
                                                float *__restrict__ out)
{
    __shared__ float acc[4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l = blockIdx.x * 64 + lane;
    float s = 0.f;
    if (l < h) {
        int r = wave;
        for (; r + 12 < rows; r += 16) {
            const float a0 = part[(size_t)r * h + l], a1 = part[(size_t)(r + 4) * h + l];
            const float a2 = part[(size_t)(r + 8) * h + l], a3 = part[(size_t)(r + 12) * h + l];
            s += a0; s += a1; s += a2; s += a3;
        }
        for (; r < rows; r += 4) s += part[(size_t)r * h + l];
    }
    acc[wave][lane] = s;
    __syncthreads();
    if (wave == 0 && l < h) out[l] = ((acc[0][lane] + acc[1][lane]) + acc[2][lane]) + acc[3][lane];
}

// 64 x 64 tiles through LDS; rows past R (up to Rp) are written as zero.  bf16 with
// 16-byte accesses on both sides when the row lengths allow (C % 8 == 0 and Rp % 8 ==
// 0, always true here): a lane loads 8 consecutive elements of a source row and
// stores 8 consecutive elements of a destination row, gathered from 8 LDS rows.
template <typename TIO>
__global__ __launch_bounds__(256) void k_transpose(const TIO *__restrict__ src, TIO *__restrict__ dst,
                                                   int R, int C, int Rp, int pitch, size_t bstride)
{
    __shared__ float tile[64][65];
    const int b = blockIdx.z;
    const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
    const TIO *S = src + (size_t)b * bstride;
    TIO *D = dst + (size_t)b * C * Rp;
    // Load: 64 rows x 8 chunks of 8 elements; thread i takes chunk i % 8 of rows i / 8
    // and i / 8 + 32.
    const int ck = threadIdx.x & 7, rr = threadIdx.x >> 3;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = rr + 32 * i, gr = r0 + r, gc = c0 + ck * 8;
        float v[8];
        if (gr < R && gc < C) {
            Vec8<TIO>::load(S + (size_t)gr * pitch + gc, v);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) tile[r][ck * 8 + e] = v[e];
    }
    __syncthreads();
    // Store: destination row gc = c0 + cc holds tile column cc; thread i writes chunk
    // i % 8 (8 consecutive r) of columns i / 8 and i / 8 + 32.
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int cc = rr + 32 * i, gc = c0 + cc, gr = r0 + ck * 8;
        if (gc >= C || gr >= Rp) continue;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = tile[ck * 8 + e][cc];
        Vec8<TIO>::store(D + (size_t)gc * Rp + gr, v);
    }
}

__device__ __forceinline__ float gelu_erf_f(float v) {
    return 0.5f * v * erfcf(-v * 0.70710678118654752f);
}
__device__ __forceinline__ float gelu_erf_grad(float v) {
    return 0.5f * erfcf(-v * 0.70710678118654752f) + v * 0.39894228040143268f * expf(-0.5f * v * v);
}
__device__ __forceinline__ float gelu_tanh_f(float v) {
    return 0.5f * v * (1.0f + tanhf(0.79788456080286536f * (v + 0.044715f * v * v * v)));
}
__device__ __forceinline__ float gelu_tanh_grad(float v) {
    const float c = 0.79788456080286536f;
    const float th = tanhf(c * (v + 0.044715f * v * v * v));
    return 0.5f * (1.0f + th) + 0.5f * v * (1.0f - th * th) * c * (1.0f + 3.0f * 0.044715f * v * v);
}

// One thread per 8 consecutive activation columns of one row.
template <int ACT, typename TIO>
__global__ __launch_bounds__(256) void k_act_bwd(size_t rows, int fs, const TIO *__restrict__ A,
                                                 const TIO *__restrict__ dY, TIO *__restrict__ da,
                                                 TIO *__restrict__ Y)
{
    constexpr bool GLU = ACT == CAAT_SWIGLU;
    const int F1 = GLU ? 2 * fs : fs;
    const int cpr = fs / 8;
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= rows * cpr) return;
    const size_t row = i / cpr;
    const int k0 = (int)(i - row * cpr) * 8;
    float a[8], dy[8], y[8], d0[8];
    Vec8<TIO>::load(A + row * F1 + k0, a);
    Vec8<TIO>::load(dY + row * fs + k0, dy);
    if (GLU) {
        float u[8], du[8];
        Vec8<TIO>::load(A + row * F1 + fs + k0, u);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float sg = 1.0f / (1.0f + expf(-a[e]));
            const float si = a[e] * sg;
            d0[e] = dy[e] * u[e] * sg * (1.0f + a[e] * (1.0f - sg));
            du[e] = dy[e] * si;
            y[e] = si * u[e];
        }
        Vec8<TIO>::store(da + row * F1 + fs + k0, du);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (ACT == CAAT_GELU) {
                d0[e] = dy[e] * gelu_erf_grad(a[e]);
                y[e] = gelu_erf_f(a[e]);
            } else {
                d0[e] = dy[e] * gelu_tanh_grad(a[e]);
                y[e] = gelu_tanh_f(a[e]);
            }
        }
    }
    Vec8<TIO>::store(da + row * F1 + k0, d0);
    Vec8<TIO>::store(Y + row * fs + k0, y);
}

template <typename TIO>
__global__ __launch_bounds__(256) void k_add(TIO *__restrict__ dst, const TIO *__restrict__ src,
                                             size_t n8)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n8) return;
    float x[8], y[8];
    Vec8<TIO>::load(dst + i * 8, x);
    Vec8<TIO>::load(src + i * 8, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] += y[e];
    Vec8<TIO>::store(dst + i * 8, x);
}

template <typename TIO>
hipError_t act_bwd_t(int act, size_t rows, int fs, const void *A, const void *dY, void *da,
                     void *Y, hipStream_t s) {
    const size_t n = rows * (size_t)(fs / 8);
    const dim3 grid((unsigned)((n + 255) / 256)), block(256);
    const TIO *a = reinterpret_cast<const TIO *>(A), *d = reinterpret_cast<const TIO *>(dY);
    TIO *o = reinterpret_cast<TIO *>(da), *y = reinterpret_cast<TIO *>(Y);
    switch (act) {
    case CAAT_GELU: hipLaunchKernelGGL((k_act_bwd<CAAT_GELU, TIO>), grid, block, 0, s, rows, fs, a, d, o, y); break;
    case CAAT_GELU_TANH: hipLaunchKernelGGL((k_act_bwd<CAAT_GELU_TANH, TIO>), grid, block, 0, s, rows, fs, a, d, o, y); break;
    default: hipLaunchKernelGGL((k_act_bwd<CAAT_SWIGLU, TIO>), grid, block, 0, s, rows, fs, a, d, o, y); break;
    }
    return hipGetLastError();
}

}  // namespace

int psync_bwd_blocks(int T) { return T < BWD_MAX_BLOCKS ? T : BWD_MAX_BLOCKS; }

hipError_t psync_norm_bwd(const PsyncBwdArgs &a, int dtype, hipStream_t s) {
    if (dtype == CAAT_BF16)
        return a.norm == CAAT_LAYERNORM ? launch_bwd<CAAT_LAYERNORM, __bf16>(a, s)
                                        : launch_bwd<CAAT_RMSNORM, __bf16>(a, s);
    return a.norm == CAAT_LAYERNORM ? launch_bwd<CAAT_LAYERNORM, float>(a, s)
                                    : launch_bwd<CAAT_RMSNORM, float>(a, s);
}

hipError_t colsum_f32(const float *part, int rows, int h, float *out, hipStream_t s) {
    hipLaunchKernelGGL(k_colsum, dim3((h + 63) / 64), dim3(256), 0, s, part, rows, h, out);
    return hipGetLastError();
}

hipError_t transpose(const void *src, void *dst, int B, int R, int C, int Rp, int dtype,
                     hipStream_t s) {
    return transpose_strided(src, dst, B, R, C, Rp, C, (size_t)R * C, dtype, s);
}

hipError_t transpose_strided(const void *src, void *dst, int B, int R, int C, int Rp, int pitch,
                             size_t bstride, int dtype, hipStream_t s) {
    const dim3 grid((C + 63) / 64, (Rp + 63) / 64, B), block(256);
    if (dtype == CAAT_BF16)
        hipLaunchKernelGGL(k_transpose<__bf16>, grid, block, 0, s,
                           reinterpret_cast<const __bf16 *>(src), reinterpret_cast<__bf16 *>(dst),
                           R, C, Rp, pitch, bstride);
    else
        hipLaunchKernelGGL(k_transpose<float>, grid, block, 0, s,
                           reinterpret_cast<const float *>(src), reinterpret_cast<float *>(dst),
                           R, C, Rp, pitch, bstride);
    return hipGetLastError();
}

hipError_t act_backward(int act, int dtype, size_t rows, int fs, const void *A, const void *dY,
                        void *da, void *Y, hipStream_t s) {
    return dtype == CAAT_BF16 ? act_bwd_t<__bf16>(act, rows, fs, A, dY, da, Y, s)
                              : act_bwd_t<float>(act, rows, fs, A, dY, da, Y, s);
}

hipError_t add_inplace(void *dst, const void *src, size_t n, int dtype, hipStream_t s) {
    const size_t n8 = n / 8;
    const dim3 grid((unsigned)((n8 + 255) / 256)), block(256);
    if (dtype == CAAT_BF16)
        hipLaunchKernelGGL(k_add<__bf16>, grid, block, 0, s, reinterpret_cast<__bf16 *>(dst),
                           reinterpret_cast<const __bf16 *>(src), n8);
    else
        hipLaunchKernelGGL(k_add<float>, grid, block, 0, s, reinterpret_cast<float *>(dst),
                           reinterpret_cast<const float *>(src), n8);
    return hipGetLastError();
}

}  // namespace caat
