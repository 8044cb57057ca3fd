// Row helpers shared by the K3 kernels and their backward: 8-element vector loads and
// stores of one 16-byte (bf16) or 32-byte (fp32) chunk, and fixed-order wave / block sums.
#pragma once

#include "caat_internal.h"

namespace caat {
namespace {

// Nontemporal 16-byte load and store (global_load / global_store ... nt), for streams that
// a launch touches once and that no cache holds: on the 7B prefill K3 (1.9 GB moved per
// launch) they take 3-8 % off the launch.  The T = 1 decode K3, whose rows a previous
// kernel has just written, and the backward's norm derivative measured slower with them,
// so the other helpers keep the ordinary forms.
typedef unsigned u32x4n __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4n ld_nt(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4n *>(p));
}
__device__ __forceinline__ void st_nt(void *p, u32x4n v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4n *>(p));
}

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
    static __device__ __forceinline__ void store_nt(__bf16 *p, const float (&v)[8]) {
        typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
        bf16x8 b;
#pragma unroll
        for (int i = 0; i < 8; ++i) b[i] = static_cast<__bf16>(v[i]);
        st_nt(p, __builtin_bit_cast(u32x4n, b));
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
    static __device__ __forceinline__ void store_nt(float *p, const float (&v)[8]) {
        typedef float f32x4n __attribute__((ext_vector_type(4)));
        const f32x4n a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
        st_nt(p, __builtin_bit_cast(u32x4n, a));
        st_nt(p + 4, __builtin_bit_cast(u32x4n, b));
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
    __device__ __forceinline__ void load_nt(const __bf16 *p) {
        const u32x4n x = ld_nt(p);
        u = make_uint4(x[0], x[1], x[2], x[3]);
    }
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
    __device__ __forceinline__ void load_nt(const float *p) {
        const u32x4n x = ld_nt(p), y = ld_nt(p + 4);
        a = make_float4(__uint_as_float(x[0]), __uint_as_float(x[1]), __uint_as_float(x[2]),
                        __uint_as_float(x[3]));
        b = make_float4(__uint_as_float(y[0]), __uint_as_float(y[1]), __uint_as_float(y[2]),
                        __uint_as_float(y[3]));
    }
    __device__ __forceinline__ void unpack(float (&v)[8]) const {
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
};

}  // namespace
}  // namespace caat
