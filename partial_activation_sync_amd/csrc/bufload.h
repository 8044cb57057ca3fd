// Buffer-descriptor loads shared by the MFMA kernels (gfx950).
//
// Every operand is read through a raw buffer descriptor whose range check turns any byte
// offset at or past its record count into a zero read: rows past a matrix, padding slots
// and K tails need no branch.  OOB is an offset past every range this library builds
// (all ranges stay below 2^31 bytes).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace caat {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t OOB = 0x80000000u;   // byte offset past every buffer's range
constexpr int RSRC_WORD3 = 0x00020000;  // gfx9 buffer descriptor: 32-bit dword format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                             RSRC_WORD3);
}

// 16 bytes per lane from a buffer straight into LDS (no registers): lane l of the wave
// writes lds + 16 l, so the 64 lanes of one instruction fill 1 KB of consecutive LDS.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, uint4 *lds, uint32_t voff,
                                           uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void *)lds, 16, voff, soff, 0, 0);
}

// load_lds16 with a cache policy (2: nontemporal, for data read once).
template <int CPOL>
__device__ __forceinline__ void load_lds16_pol(__amdgpu_buffer_rsrc_t r, uint4 *lds, uint32_t voff,
                                               uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void *)lds, 16, voff, soff, 0, CPOL);
}

// 16 bytes per lane into registers.
__device__ __forceinline__ bf16x8 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

}  // namespace caat
