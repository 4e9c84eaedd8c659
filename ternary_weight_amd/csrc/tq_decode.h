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

// Buffer resources: a 32-bit per-lane offset (VGPR) plus a wave-uniform
// offset (SGPR) from a base; a lane whose VGPR offset is at or past the
// resource's size reads zeros without touching memory.  The SGPR offset is
// kept inside the data wherever the load's result is used, since only the
// VGPR offset is certain to take part in the range check.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kOffNone = 0x80000000u;   // VGPR offset that reads zero (resources are < 2 GiB)
constexpr int kCacheNT = 2;                  // cache policy: non-temporal (streamed once)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(uint32_t)bytes, 0x00020000);
}

template <typename F, int kPolicy = 0>
__device__ __forceinline__ F buffer_load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff);
template <>
__device__ __forceinline__ u32x4 buffer_load<u32x4, 0>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
template <>
__device__ __forceinline__ u32x4 buffer_load<u32x4, kCacheNT>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kCacheNT));
}
template <>
__device__ __forceinline__ u32x2 buffer_load<u32x2, 0>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
template <>
__device__ __forceinline__ u32x2 buffer_load<u32x2, kCacheNT>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kCacheNT));
}
template <>
__device__ __forceinline__ uint32_t buffer_load<uint32_t, 0>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

// The pair-code table of the compact base-3 codec: entry e (10-bit code),
// copy c at byte offset e * 4 C + c * 4 holds bf16(v0) | bf16(v1) << 16 for
// e = (v0 mod 27) + 27 (v1 mod 27) < 729, and zero for the codes never
// written.  Lane l reads copy l % C.  C copies spread the lanes' reads over
// the banks (C = 16, 64 KiB, for one-token decode; 8, 32 KiB, where a
// smaller table lets more waves share a compute unit -- measured).
template <int C>
struct B3Table {
    static_assert(C == 8 || C == 16 || C == 32, "8, 16 or 32 copies");
    static constexpr int kCopies = C;
    static constexpr int kShift = C == 32 ? 7 : (C == 16 ? 6 : 5);   // log2(4 C)
    static constexpr int kBytes = 1024 * 4 * C;
    static __device__ __forceinline__ void fill(uint8_t* lut)
    {
        for (int i = threadIdx.x; i < 1024 * C; i += blockDim.x) {
            const uint32_t e = (uint32_t)i / C, c = (uint32_t)i % C;
            uint32_t v = 0;
            if (e < (uint32_t)TQ_B3_CODES) {
                const int a = (int)(e % 27u), b = (int)(e / 27u);
                // small integers: the fp32 value's upper half is the exact bf16
                v = (__float_as_uint((float)(a > 13 ? a - 27 : a)) >> 16) |
                    (__float_as_uint((float)(b > 13 ? b - 27 : b)) & 0xFFFF0000u);
            }
            *(LDS_AS uint32_t*)((LDS_AS uint8_t*)lut + e * (4 * C) + c * 4) = v;
        }
    }
    static __device__ __forceinline__ uint32_t copy_offset() { return (uint32_t)(threadIdx.x % C) * 4u; }
};

// The combined-digit table of the codec's two-bit digit planes (three
// planes, plane k weighing 3^(2 - k)): a column's 6-bit code g holds plane
// k's digit code at bits 2k, 2k + 1 (01 = +1, 10 = -1, 00 and 11 = 0), and
// the bf16 at byte 2 g is the column's combined value 9 d0 + 3 d1 + d2, an
// integer in [-13, 13], exact in bf16 (d3 card, "Quantization details").
// 128 bytes: 32 dwords, one per bank, so no two lanes' reads conflict.
struct D3Table {
    static constexpr int kBytes = 128;
    static __device__ __forceinline__ int digit(uint32_t c) { return c == 1u ? 1 : (c == 2u ? -1 : 0); }
    static __device__ __forceinline__ void fill(uint8_t* lut)
    {
        const uint32_t g = threadIdx.x;
        if (g < 64) {
            const int v = 9 * digit(g & 3u) + 3 * digit((g >> 2) & 3u) + digit((g >> 4) & 3u);
            // a small integer: the fp32 value's upper half is the exact bf16
            *(LDS_AS uint16_t*)((LDS_AS uint8_t*)lut + 2 * g) = (uint16_t)(__float_as_uint((float)v) >> 16);
        }
    }
};

__device__ __forceinline__ float f16_to_f32(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }

}  // namespace tqk
