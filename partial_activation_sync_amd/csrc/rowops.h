// Row helpers shared by the K3 kernels and their backward: 8-element vector loads and
// stores of one 16-byte (bf16) or 32-byte (fp32) chunk, and fixed-order wave / block sums.
#pragma once

#include "caat_internal.h"

namespace caat {
namespace {

template <typename TIO> struct Vec8;

template <> struct Vec8<__bf16> {
    static __device__ __forceinline__ void load(const __bf16 *p, float (&v)[8]) {
        uint4 u = *reinterpret_cast<const uint4 *>(p);
        uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void store(__bf16 *p, const float (&v)[8]) {
        typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
        bf16x8 b;
#pragma unroll
        for (int i = 0; i < 8; ++i) b[i] = static_cast<__bf16>(v[i]);
        *reinterpret_cast<bf16x8 *>(p) = b;
    }
};

template <> struct Vec8<float> {
    static __device__ __forceinline__ void load(const float *p, float (&v)[8]) {
        float4 a = *reinterpret_cast<const float4 *>(p);
        float4 b = *reinterpret_cast<const float4 *>(p + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    static __device__ __forceinline__ void store(float *p, const float (&v)[8]) {
        *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4 *>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Sums v[g] (g < NV) over the whole block in a fixed order; red is LDS with room for
// (blockDim / 64) x NV floats.  A caller that reuses red must synchronize first.
template <int NV>
__device__ __forceinline__ void block_sum(float (&v)[NV], float *red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
#pragma unroll
    for (int g = 0; g < NV; ++g) v[g] = wave_sum(v[g]);
    if (lane == 0) {
#pragma unroll
        for (int g = 0; g < NV; ++g) red[wave * NV + g] = v[g];
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < NV; ++g) {
        float s = 0.f;
        for (int w = 0; w < nwaves; ++w) s += red[w * NV + g];
        v[g] = s;
    }
}

// One 8-element chunk kept in its storage format (4 VGPRs for bf16) and unpacked to fp32
// where it is used.
template <typename TIO> struct Raw;
template <> struct Raw<__bf16> {
    uint4 u;
    __device__ __forceinline__ void load(const __bf16 *p) { u = *reinterpret_cast<const uint4 *>(p); }
    __device__ __forceinline__ void zero() { u = make_uint4(0, 0, 0, 0); }
    __device__ __forceinline__ void unpack(float (&v)[8]) const {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
};
template <> struct Raw<float> {
    float4 a, b;
    __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
    __device__ __forceinline__ void load(const float *p) {
        a = *reinterpret_cast<const float4 *>(p);
        b = *reinterpret_cast<const float4 *>(p + 4);
    }
    __device__ __forceinline__ void unpack(float (&v)[8]) const {
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
};

}  // namespace
}  // namespace caat
