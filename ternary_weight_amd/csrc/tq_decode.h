#pragma once
// libtq: trit decode shared by the decode (vector ALU) and prefill (MFMA)
// kernels.  Codes are 2 bits per trit, 00 = 0, 01 = +1, 10 = -1, 11 reads as
// 0; a dword holds 16 consecutive columns, column 4p + b in byte b, bits 2p.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define CONST_AS __attribute__((address_space(4)))
#define GLOBAL_AS __attribute__((address_space(1)))
#define LDS_AS __attribute__((address_space(3)))
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

namespace tqk {

// Loads of wave-uniform data through the constant address space, which the
// compiler serves with scalar (SMEM) loads into SGPRs.
template <typename T>
__device__ __forceinline__ T ld_uniform(const T* p)
{
    return *(const CONST_AS T*)p;
}

__device__ __forceinline__ uint32_t ld_uniform_u32(const void* base, int64_t dword)
{
    return ((const CONST_AS uint32_t*)base)[dword];
}

template <typename T>
__device__ __forceinline__ T ld_uniform_struct(const T* p)
{
    static_assert(sizeof(T) % 4 == 0, "dword-sized struct");
    T v;
    uint32_t* d = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 4); ++i) d[i] = ld_uniform_u32(p, i);
    return v;
}

// int8 trits of columns 4j..4j+3 (j = 0..3) of a 16-column dword of codes.
__device__ __forceinline__ void decode_i8(uint32_t w, uint32_t t[4])
{
    const uint32_t w4 = w >> 4;
    // bits 0..1 of each byte: selector 0,1,2,3 -> bytes of 0x00FF0100 = 0, +1, -1, 0
    t[0] = __builtin_amdgcn_perm(0u, 0x00FF0100u, w & 0x03030303u);
    t[2] = __builtin_amdgcn_perm(0u, 0x00FF0100u, w4 & 0x03030303u);
    // bits 2..3 of each byte: selector 0 -> 0x00, 4 -> 0x01, 8 -> sign of 0x8000 -> 0xFF, 12 -> 0
    t[1] = __builtin_amdgcn_perm(0x00000001u, 0x00008000u, w & 0x0C0C0C0Cu);
    t[3] = __builtin_amdgcn_perm(0x00000001u, 0x00008000u, w4 & 0x0C0C0C0Cu);
}

__device__ __forceinline__ float f16_to_f32(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }

}  // namespace tqk
