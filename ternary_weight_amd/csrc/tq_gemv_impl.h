#pragma once
// libtq: decode kernels (M <= 16) -- tq_gemv and tq_gemv_grouped.
//
// What is computed is the definition in tq.h: per output row, each trit plane
// adds or subtracts the activations of its nonzero trits, with no multiply by
// a weight in the inner loop (QORA-LLM-2B page), per-group sums are
// scaled once at the group's end (sasori page, "K and g"), a per-tensor scale
// once at the very end (QORA-LLM-2B, "Ternary GEMV (No Multiplication)").
//
// Mapping onto CDNA4.  One wave64 owns a block of 64 output rows, one row per
// lane, so a lane's 16-byte slot of the blob is 64 trits of its own row and a
// wave-wide load is 1 KiB of contiguous codes (see tq_layout.h).  All lanes
// of a wave read the same activations, so x is fetched with scalar loads into
// SGPRs and fed to the vector ALU as a uniform operand; no LDS staging and no
// cross-lane reduction are needed.  The waves of a workgroup split the columns
// of the row block (whole groups each) and add their partial sums in LDS in a
// fixed order at the end.
//
// Trit decode, per dword of codes (16 trits):
//  int8   (w >> 4p) masked to two bits per byte and mapped to {0, +1, -1}
//         bytes by one v_perm_b32 each (a byte lookup table in the selector's
//         source operands; for the bits-2..3 field the selector value 8
//         replicates the sign bit of a source byte, which yields 0xFF), then
//         one v_dot4_i32_i8 against four int8 activations: about 13 VALU ops
//         per 16 trits.
//  bf16   a table in LDS maps each code byte (four trits) to four bf16 values
//         {0, +1, -1} (8 bytes); one v_perm_b32 builds the byte address from
//         the code byte and the lane's copy offset, one 8-byte LDS read fetches
//         the four values and two v_dot2_f32_bf16 accumulate them against the
//         matching activation pairs, which the scalar unit assembles with
//         s_pack.  The table is 256 entries x 32 copies (64 KiB): 32 lanes read
//         32 different copies, so a wave's read has no bank conflicts.
//  fp32   int8 decode as above, converted per trit and accumulated with fma
//         (t in {-1, 0, 1}, so each fma is an exact add, subtract or no-op).
//  codec, compact base-3 codes (CODEBOOK_B3, bf16 activations): a table in
//         LDS maps each 10-bit pair code to the two weights' values as a
//         bf16 pair (exact: integers in [-13, 13]); one field extract, one
//         address op and one 4-byte LDS read per two columns, then one
//         v_dot2_f32_bf16 against the activation pair of the same two
//         columns (consecutive, so x needs no rearranging).  The digits'
//         weights 9, 3, 1 are in the table values, so a group's sum is scaled
//         once by its codebook entry.  1024 entries x 16 copies (64 KiB)
//         for one token, 8 (32 KiB) for several.
#include "tq_internal.h"
#include "tq_decode.h"

#include <algorithm>
#include <type_traits>

namespace tqk {

// Tuning constants (measured on MI355X).
#ifndef TQ_Q8_HELD
#define TQ_Q8_HELD 2          // fp32 activation vectors held per thread while quantising
#endif
#ifndef TQ_Q8_EARLY_LOADS
#define TQ_Q8_EARLY_LOADS 0   // issue the first code loads before quantising
#endif
#ifndef TQ_DEPTH_K1
#define TQ_DEPTH_K1 2         // chunks in flight per wave, one plane
#endif
#ifndef TQ_DEPTH_KN
#define TQ_DEPTH_KN 1         // chunks in flight per wave, several planes
#endif
#ifndef TQ_DEPTH_BF16
#define TQ_DEPTH_BF16 2       // chunks in flight per wave, bf16 activations (table decode)
#endif

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }

template <int XT>
struct XUnit;   // activations of one 16-column unit of one token

template <>
struct XUnit<TQ_I8> {
    uint32_t v[4];
    __device__ __forceinline__ void load(const void* x, int64_t elem)
    {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = ld_uniform_u32(x, (elem >> 2) + j);
    }
};
template <>
struct XUnit<TQ_BF16> {
    uint32_t v[8];
    __device__ __forceinline__ void load(const void* x, int64_t elem)
    {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = ld_uniform_u32(x, (elem >> 1) + j);
    }
};
template <>
struct XUnit<TQ_F32> {
    uint32_t v[16];
    __device__ __forceinline__ void load(const void* x, int64_t elem)
    {
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = ld_uniform_u32(x, elem + j);
    }
};

// fp32 activations quantised to int8 inside the kernel: staged in LDS.
template <>
struct XUnit<TQ_F32_Q8> : XUnit<TQ_I8> {
    __device__ __forceinline__ void load(const void* xq_lds, int64_t elem)
    {
        const LDS_AS uint32_t* p = (const LDS_AS uint32_t*)xq_lds + (elem >> 2);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = p[j];
    }
};

template <int XT>
struct AccT { using type = float; };
template <>
struct AccT<TQ_I8> { using type = int; };
template <>
struct AccT<TQ_F32_Q8> { using type = int; };

// The trits of one 16-column code dword, decoded once and shared by every
// token: int8 values (integer and fp32 paths), or the four 8-byte entries of
// the bf16 table (below).
template <int XT>
struct Trits { uint32_t t[4]; };
template <>
struct Trits<TQ_BF16> { uint64_t t[4]; };

// acc += sum over the 16 columns of one code dword of t * x.
__device__ __forceinline__ void accum(const Trits<TQ_I8>& t, const XUnit<TQ_I8>& x, int& acc)
{
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_sdot4((int)t.t[j], (int)x.v[j], acc, false);
}

// bf16 activations: a lookup table in LDS maps one code byte (the trits of
// columns b, 4+b, 8+b, 12+b of a 16-column dword) to four bf16 values in
// {0, +1, -1}, as the pairs (t_b, t_4+b) and (t_8+b, t_12+b).  The table has
// 32 copies, lane l reading copy l % 32, so that the 8-byte reads of a wave
// never share a bank.  Entry e, copy c sits at byte offset e * 256 + c * 8, so
// one v_perm_b32 builds the address: byte 1 = the code byte, byte 0 = c * 8.
constexpr int kLutBytes = 256 * 256;

struct BfPairs {   // activation pairs of one 16-column unit, matching the table's pairs
    uint32_t a[4], b[4];
};

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Two 16-bit halves of wave-uniform dwords into one (the scalar unit's
// s_pack_ll_b32_b16 and s_pack_hh_b32_b16): low halves, or high halves, of a
// and b.
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b)
{
    return __builtin_bit_cast(uint32_t, u16x2{(unsigned short)a, (unsigned short)b});
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b)
{
    // written out: the compiler forms it as two shifts and s_pack_ll.  The
    // operands are uniform; readfirstlane only moves one the compiler keeps
    // in a VGPR to an SGPR (and vanishes when it is in one already).
    uint32_t r;
    asm("s_pack_hh_b32_b16 %0, %1, %2"
        : "=s"(r)
        : "s"(__builtin_amdgcn_readfirstlane((int)a)), "s"(__builtin_amdgcn_readfirstlane((int)b)));
    return r;
}

__device__ __forceinline__ BfPairs bf_pairs(const XUnit<TQ_BF16>& x)
{
    // x.v[j] holds columns 2j (low half) and 2j+1 (high half)
    BfPairs p;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint32_t x0 = x.v[b >> 1], x4 = x.v[2 + (b >> 1)], x8 = x.v[4 + (b >> 1)], x12 = x.v[6 + (b >> 1)];
        if (b & 1) {
            p.a[b] = pack_hi(x0, x4);
            p.b[b] = pack_hi(x8, x12);
        } else {
            p.a[b] = pack_lo(x0, x4);
            p.b[b] = pack_lo(x8, x12);
        }
    }
    return p;
}

__device__ __forceinline__ Trits<TQ_BF16> lut_lookup(uint32_t w, const LDS_AS uint8_t* lut, uint32_t copyoff)
{
    Trits<TQ_BF16> r;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint32_t addr = __builtin_amdgcn_perm(w, copyoff, 0x0C0C0400u | ((4u + b) << 8));
        r.t[b] = *(const LDS_AS uint64_t*)(lut + addr);
    }
    return r;
}

// One token: the table reads interleaved with their dot products.
__device__ __forceinline__ void accum_lut(uint32_t w, const BfPairs& xp, float& acc, const LDS_AS uint8_t* lut,
                                          uint32_t copyoff)
{
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint32_t addr = __builtin_amdgcn_perm(w, copyoff, 0x0C0C0400u | ((4u + b) << 8));
        const uint64_t t = *(const LDS_AS uint64_t*)(lut + addr);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, (uint32_t)t),
                                              __builtin_bit_cast(bf16x2_t, xp.a[b]), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, (uint32_t)(t >> 32)),
                                              __builtin_bit_cast(bf16x2_t, xp.b[b]), acc, false);
    }
}

__device__ __forceinline__ void accum(const Trits<TQ_BF16>& t, const BfPairs& xp, float& acc)
{
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint32_t t0 = (uint32_t)t.t[b], t1 = (uint32_t)(t.t[b] >> 32);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, t0),
                                              __builtin_bit_cast(bf16x2_t, xp.a[b]), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, t1),
                                              __builtin_bit_cast(bf16x2_t, xp.b[b]), acc, false);
    }
}

// Fill the table (all threads of the workgroup; the caller synchronises).
__device__ __forceinline__ void fill_bf16_lut(uint8_t* lut)
{
    for (int i = threadIdx.x; i < 256 * 32; i += blockDim.x) {
        const uint32_t e = (uint32_t)i >> 5, c = (uint32_t)i & 31u;
        uint32_t h[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t code = (e >> (2 * q)) & 3u;
            h[q] = code == 1u ? 0x3F80u : (code == 2u ? 0xBF80u : 0u);
        }
        *(LDS_AS uint64_t*)(lut + e * 256 + c * 8) =
            (uint64_t)(h[0] | (h[1] << 16)) | ((uint64_t)(h[2] | (h[3] << 16)) << 32);
    }
}

// Field i (columns 2i, 2i + 1) of 16-column unit d of a CODEBOOK_B3 chunk
// stream (ten dwords w), as its table address.
template <int d, int i, int SHIFT>
__device__ __forceinline__ uint32_t b3_addr(const u32x4 (&w)[3], uint32_t copyoff)
{
    constexpr int bit = 80 * d + 10 * i, D = bit >> 5, S = bit & 31;
    uint32_t f;
    if constexpr (S <= 22) {
        f = __builtin_amdgcn_ubfe(w[D >> 2][D & 3], S, 10);
    } else {
        constexpr int D1 = D + 1;
        f = __builtin_amdgcn_alignbit(w[D1 >> 2][D1 & 3], w[D >> 2][D & 3], S) & 0x3FFu;
    }
    return (f << SHIFT) | copyoff;
}

__device__ __forceinline__ void accum(const Trits<TQ_F32>& t, const XUnit<TQ_F32>& x, float& acc)
{
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float tf = (float)(int8_t)(t.t[j] >> (8 * b));
            acc = fmaf(tf, __uint_as_float(x.v[4 * j + b]), acc);
        }
    }
}

// Factor of the decoded trit values (all paths decode exactly +-1).
template <int XT>
__device__ __forceinline__ constexpr float enc_scale() { return 1.0f; }

template <int K>
__device__ __forceinline__ int codec_combine(const int (&p)[K])
{
    int v = 0;
#pragma unroll
    for (int k = 0; k < K; ++k) v = v * 3 + p[k];
    return v;
}

template <int K>
__device__ __forceinline__ float codec_combine(const float (&p)[K])
{
    float v = p[0];
#pragma unroll
    for (int k = 1; k < K; ++k) v = fmaf(v, 3.0f, p[k]);
    return v;
}

// Code (and scale) registers of one 64-column chunk.
template <int K, int LAYOUT>
struct Slot {
    // CODEBOOK_B3: the chunk's 320-bit stream in w[0], w[1] and w[2].xy
    u32x4 w[LAYOUT == TQ_SCALE_CODEBOOK_B3 ? 3 : K];
    uint32_t sw[LAYOUT == TQ_SCALE_TENSOR ? 1 : K][2];
};

template <int XT>
struct XChunk {   // activations of one 64-column chunk of one token (SGPRs, or VGPRs from LDS)
    static constexpr int kD = (XT == TQ_I8 || XT == TQ_F32_Q8) ? 16 : (XT == TQ_BF16 ? 32 : 64);
    uint32_t v[kD];
    __device__ __forceinline__ void load(const void* x, int64_t elem)
    {
        if (XT == TQ_F32_Q8) {
            const LDS_AS uint32_t* p = (const LDS_AS uint32_t*)x + (elem >> 2);
#pragma unroll
            for (int j = 0; j < kD; ++j) v[j] = p[j];
            return;
        }
        const int64_t dw = XT == TQ_I8 ? (elem >> 2) : (XT == TQ_BF16 ? (elem >> 1) : elem);
#pragma unroll
        for (int j = 0; j < kD; ++j) v[j] = ld_uniform_u32(x, dw + j);
    }
    __device__ __forceinline__ XUnit<XT> unit(int d) const
    {
        XUnit<XT> u;
        constexpr int n = kD / 4;
#pragma unroll
        for (int j = 0; j < n; ++j) u.v[j] = v[d * n + j];
        return u;
    }
};

// One row block (64 rows) of one problem, columns split across `nwaves` waves.
// kDepth: chunks in flight per wave (0: the decode kernels' tuned depth).
template <int XT, int LAYOUT, int K, int MT, int kDepth = 0>
struct RowBlock {
    using A = typename AccT<XT>::type;
    static constexpr bool kGroup = LAYOUT != TQ_SCALE_TENSOR;
    // the codec's compact base-3 codes: one combined value per weight (K = 1
    // here), decoded through the pair-code table (bf16 activations only)
    static constexpr bool kB3 = LAYOUT == TQ_SCALE_CODEBOOK_B3;
    static constexpr bool kCb = LAYOUT == TQ_SCALE_CODEBOOK || kB3;
    using B3T = B3Table<MT == 1 ? 16 : 8>;   // pair-code table (one token: more copies, fewer conflicts)
    static_assert(!kB3 || (K == 1 && XT == TQ_BF16), "compact base-3 codes: one combined plane, bf16 activations");
    // chunks in flight per wave (codes of K planes each)
    static constexpr int D = kDepth > 0 ? kDepth
                           : (MT > 1 ? 1 : (XT == TQ_BF16 ? TQ_DEPTH_BF16 : (K == 1 ? TQ_DEPTH_K1 : TQ_DEPTH_KN)));
    static_assert(XT != TQ_BF16 || sizeof(typename AccT<XT>::type) == 4, "bf16 accumulates in fp32");
    // activations are prefetched a chunk ahead for one token (SGPR budget);
    // not with an explicit depth (the chain reads its x from LDS as it goes)
    static constexpr bool kXPre = kDepth == 0 && MT == 1 && (XT == TQ_I8 || XT == TQ_F32_Q8);

    const tq_prob_dev& P;
    const int rb, lane;
    const void* xsrc;     // activations: global x, or the LDS copy quantised to int8
    const void* xrow[MT];  // each token's row of them (the loads then add only the column)
    const LDS_AS uint8_t* lut;   // bf16 trit table (TQ_BF16)
    uint32_t copyoff;
    A p[MT][K];
    float out[MT];
    const uint8_t* cbase;   // this row block's codes
    const uint8_t* sbase;   // this row block's scale words

    __device__ __forceinline__ RowBlock(const tq_prob_dev& P_, int rb_, const void* xsrc_, const uint8_t* lut_)
        : P(P_), rb(rb_), lane(threadIdx.x & 63), xsrc(xsrc_), lut((const LDS_AS uint8_t*)lut_),
          copyoff(kB3 ? B3T::copy_offset() : (uint32_t)(threadIdx.x & 31) * 8u)
    {
        constexpr int64_t kXBytes = XT == TQ_F32 ? 4 : (XT == TQ_BF16 ? 2 : 1);   // TQ_F32_Q8: the int8 copy
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            out[m] = 0.0f;
#pragma unroll
            for (int k = 0; k < K; ++k) p[m][k] = 0;
            // a token past the problem's count reads its last token's row
            // (the token loop stops before it)
            if (MT > 1) xrow[m] = (const uint8_t*)xsrc + (int64_t)std::min(m, P.M - 1) * P.Kin * kXBytes;
        }
        cbase = (const uint8_t*)P.codes +
                (kB3 ? (int64_t)rb * P.NC * TQ_B3_CHUNK_BYTES : (int64_t)rb * P.NC * K * TQ_ROWS * 16);
        sbase = (const uint8_t*)P.scales + (kCb ? (int64_t)rb * P.NID : (int64_t)rb * P.NGD * K) * TQ_ROWS * 4;
    }

    // A buffer resource over `bytes` bytes at `base + off` (no bytes when the
    // load is not needed: its lanes then read zeros and touch no memory).
    static __device__ __forceinline__ __amdgpu_buffer_rsrc_t window(const uint8_t* base, int64_t off, bool need,
                                                                  int bytes)
    {
        return rsrc(base + off, need ? bytes : 0);
    }

    // Codes of chunk c (K planes) and the scale words needed by the groups
    // that end inside it.  Every load is issued whatever c is, so that no
    // load sits under a branch (the compiler would then wait for all loads
    // in flight at the join); chunks at or past c1 read zeros.
    __device__ __forceinline__ void load_slot(int c_, Slot<K, LAYOUT>& s) const
    {
        const int c = __builtin_amdgcn_readfirstlane(c_);   // wave-uniform: keep its arithmetic scalar
        const bool valid = c < c1_;
        if constexpr (kB3) {
            const __amdgpu_buffer_rsrc_t rc = window(cbase, (int64_t)c * TQ_B3_CHUNK_BYTES, valid, TQ_B3_CHUNK_BYTES);
            s.w[0] = buffer_load<u32x4, kCacheNT>(rc, lane * 16, 0);
            s.w[1] = buffer_load<u32x4, kCacheNT>(rc, lane * 16, 1024);
            const u32x2 t = buffer_load<u32x2, kCacheNT>(rc, lane * 8, 2048);
            s.w[2] = u32x4{t[0], t[1], 0u, 0u};
        } else {
            const __amdgpu_buffer_rsrc_t rc = window(cbase, (int64_t)c * K * TQ_ROWS * 16, valid, K * TQ_ROWS * 16);
#pragma unroll
            for (int k = 0; k < K; ++k) s.w[k] = buffer_load<u32x4, kCacheNT>(rc, lane * 16, k * TQ_ROWS * 16);
        }
        constexpr int kWordRow = TQ_ROWS * 4;   // one scale word per row of the block
        if (LAYOUT == TQ_SCALE_GROUP_F16) {
            const int g = P.g;
            const int end = std::min((c + 1) * TQ_CHUNK, P.Kin);
            const int last_pair = ((end >> P.log2g) - 1) >> 1;
            if (g < 64) {
                const int first_pair = ((c * TQ_CHUNK) >> P.log2g) >> 1;
                const int second = std::min(first_pair + 1, last_pair);
                const __amdgpu_buffer_rsrc_t r0 = window(sbase, (int64_t)first_pair * K * kWordRow, valid, K * kWordRow);
                const __amdgpu_buffer_rsrc_t r1 = window(sbase, (int64_t)second * K * kWordRow, valid, K * kWordRow);
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    s.sw[k][0] = buffer_load<uint32_t>(r0, lane * 4, k * kWordRow);
                    s.sw[k][1] = buffer_load<uint32_t>(r1, lane * 4, k * kWordRow);
                }
            } else {
                const bool ends = (end & (g - 1)) == 0;   // a group ends in this chunk
                const __amdgpu_buffer_rsrc_t r0 =
                    window(sbase, (int64_t)last_pair * K * kWordRow, valid && ends, K * kWordRow);
#pragma unroll
                for (int k = 0; k < K; ++k) s.sw[k][0] = buffer_load<uint32_t>(r0, lane * 4, k * kWordRow);
            }
        } else if (kCb) {
            const int end = std::min((c + 1) * TQ_CHUNK, P.Kin);
            const int first_id = ((c * TQ_CHUNK) >> P.log2g) / 6;
            const int last_id = ((end >> P.log2g) - 1) / 6;
            const int second = std::min(first_id + 1, last_id);
            s.sw[0][0] = buffer_load<uint32_t>(window(sbase, (int64_t)first_id * kWordRow, valid, kWordRow), lane * 4, 0);
            s.sw[0][1] = buffer_load<uint32_t>(window(sbase, (int64_t)second * kWordRow, valid, kWordRow), lane * 4, 0);
        }
    }

    // Scale the finished group's partial sums q into out; sc: the group's
    // scale per plane (GROUP), or its codebook scale (CODEBOOK).
    __device__ __forceinline__ void apply_group(const float (&sc)[K], const A (&q)[MT][K])
    {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (LAYOUT == TQ_SCALE_GROUP_F16) {
#pragma unroll
                for (int k = 0; k < K; ++k) out[m] = fmaf(sc[k], (float)q[m][k], out[m]);
            } else {
                out[m] = fmaf(sc[0], (float)codec_combine<K>(q[m]), out[m]);
            }
        }
    }

    // Group grp ends inside chunk c: its scale, applied to p, which restarts.
    __device__ __forceinline__ void close_group(int grp, int c, const Slot<K, LAYOUT>& s, const float* cb_lds)
    {
        float sc[K];
        if (LAYOUT == TQ_SCALE_GROUP_F16) {
            int j = 0;
            if (P.g < 64) j = (grp >> 1) - (((c * TQ_CHUNK) >> P.log2g) >> 1);
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const uint32_t word = j ? s.sw[k][1] : s.sw[k][0];
                sc[k] = f16_to_f32((grp & 1) ? (word >> 16) : (word & 0xFFFFu)) * enc_scale<XT>();
            }
        } else {
            const int id = grp / 6;
            const int j = id - ((c * TQ_CHUNK) >> P.log2g) / 6;
            const uint32_t word = j ? s.sw[0][1] : s.sw[0][0];
            const uint32_t idx = (word >> (5 * (grp - 6 * id))) & 31u;
            sc[0] = cb_lds[idx] * enc_scale<XT>();
        }
        apply_group(sc, p);
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int k = 0; k < K; ++k) p[m][k] = 0;
    }

    // g = 16: unit d of chunk c is group 4 c + d.  In the chunk's words the
    // group-f16 scales of unit d are the half d % 2 of word d / 2; the
    // codebook index is field pos = (4 c) % 6 + d of the first word (of the
    // second from pos 6 on), with pos0 = (4 c) % 6.
    template <int d>
    __device__ __forceinline__ void scales_g16(const Slot<K, LAYOUT>& s, uint32_t pos0, const float* cb_lds,
                                               float (&sc)[K]) const
    {
        if (LAYOUT == TQ_SCALE_GROUP_F16) {
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const uint32_t word = s.sw[k][d >> 1];
                sc[k] = f16_to_f32((d & 1) ? (word >> 16) : (word & 0xFFFFu)) * enc_scale<XT>();
            }
        } else {
            const uint32_t pos = pos0 + d;
            const bool second = pos >= 6;
            const uint32_t word = second ? s.sw[0][1] : s.sw[0][0];
            const uint32_t idx = (word >> (5 * (second ? pos - 6 : pos))) & 31u;
            sc[0] = cb_lds[idx] * enc_scale<XT>();
        }
    }

    // Columns of chunk c: `nu` 16-column units (4 for a full chunk).
    // kG16: the group size is 16, so each unit is one group and its sums
    // start from zero in fresh registers.  kAll: the problem has all MT
    // tokens, so the token loop has no branch (with fewer, each token past
    // the count ends it).
    template <bool kFull, bool kG16, bool kAll>
    __device__ __forceinline__ void compute(int c_, int nu, const Slot<K, LAYOUT>& s, const XChunk<XT>* xc,
                                            const float* cb_lds)
    {
        const int c = __builtin_amdgcn_readfirstlane(c_);   // wave-uniform: keep its arithmetic scalar
        const uint32_t pos0 = kG16 && kCb ? (uint32_t)(4 * c) % 6u : 0u;
        const auto unit = [&](auto dc) {
            constexpr int d = decltype(dc)::value;
            if (!kFull && d >= nu) return;
            const int u = c * 4 + d;
            using TX = Trits<XT == TQ_F32_Q8 ? TQ_I8 : XT>;
            auto decode = [&](int k) {
                TX t;
                if constexpr (XT == TQ_BF16) t = lut_lookup(s.w[k][d], lut, copyoff);
                else decode_i8(s.w[k][d], t.t);
                return t;
            };
            A q[MT][K];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
#pragma unroll
                for (int k = 0; k < K; ++k) q[m][k] = kG16 ? (A)0 : p[m][k];
            }
            if constexpr (kB3) {
                // the unit's eight pair codes through the table, once for every token
                uint32_t e[8];
                const auto look = [&](auto ic) {
                    constexpr int i = decltype(ic)::value;
                    e[i] = *(const LDS_AS uint32_t*)(lut + b3_addr<d, i, B3T::kShift>(s.w, copyoff));
                };
                look(std::integral_constant<int, 0>{});
                look(std::integral_constant<int, 1>{});
                look(std::integral_constant<int, 2>{});
                look(std::integral_constant<int, 3>{});
                look(std::integral_constant<int, 4>{});
                look(std::integral_constant<int, 5>{});
                look(std::integral_constant<int, 6>{});
                look(std::integral_constant<int, 7>{});
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    if (!kAll && MT > 1 && m >= P.M) break;
                    XUnit<XT> xu;
                    if (MT == 1) xu.load(xsrc, (int64_t)u * 16);
                    else xu.load(xrow[m], (int64_t)u * 16);
                    // x dword i holds columns 2i (low half) and 2i + 1: the pair of entry i
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        q[m][0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, e[i]),
                                                                  __builtin_bit_cast(bf16x2_t, xu.v[i]), q[m][0],
                                                                  false);
                }
            } else {
            // one token: each plane decoded right before its sums; several:
            // the unit's trits decoded once, then every token's sums
            TX t[MT > 1 ? K : 1];
            if constexpr (MT > 1) {
#pragma unroll
                for (int k = 0; k < K; ++k) t[k] = decode(k);
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                if (!kAll && MT > 1 && m >= P.M) break;
                XUnit<XT> xu;
                if (kXPre && kFull) xu = xc->unit(d);
                else if (MT == 1) xu.load(xsrc, (int64_t)u * 16);
                else xu.load(xrow[m], (int64_t)u * 16);
                if constexpr (XT == TQ_BF16) {
                    const BfPairs xp = bf_pairs(xu);
#pragma unroll
                    for (int k = 0; k < K; ++k) {
                        if constexpr (MT > 1) accum(t[k], xp, q[m][k]);
                        else accum_lut(s.w[k][d], xp, q[m][k], lut, copyoff);
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < K; ++k) accum(MT > 1 ? t[k] : decode(k), xu, q[m][k]);
                }
            }
            }   // not kB3
            if constexpr (kG16) {
                float sc[K];
                scales_g16<d>(s, pos0, cb_lds, sc);
                apply_group(sc, q);
            } else {
#pragma unroll
                for (int m = 0; m < MT; ++m)
#pragma unroll
                    for (int k = 0; k < K; ++k) p[m][k] = q[m][k];
                if (kGroup) {
                    const int colend = (u + 1) * 16;
                    if ((colend & (P.g - 1)) == 0) close_group((colend >> P.log2g) - 1, c, s, cb_lds);
                }
            }
        };
        unit(std::integral_constant<int, 0>{});
        unit(std::integral_constant<int, 1>{});
        unit(std::integral_constant<int, 2>{});
        unit(std::integral_constant<int, 3>{});
    }

    Slot<K, LAYOUT> cur[D];
    int c0_, c1_, cf_;

    // Issue the loads of the first chunks (before any other set-up work).
    __device__ __forceinline__ void begin(int c0, int c1)
    {
        c0_ = c0;
        c1_ = c1;
        cf_ = std::min(c1, (P.Kin >> 4) >> 2);   // end of the chunks with all 64 columns valid
#pragma unroll
        for (int j = 0; j < D; ++j) load_slot(c0 + j, cur[j]);
    }

    __device__ __forceinline__ void run(int c0, int c1, const float* cb_lds)
    {
        begin(c0, c1);
        finish(cb_lds);
    }

    __device__ __forceinline__ void finish(const float* cb_lds)
    {
        // one copy of the loop per case, chosen once per row block
        const bool all = MT == 1 || P.M == MT;
        if (kGroup && P.g == 16) {
            if (all) run_chunks<true, true>(cb_lds);
            else run_chunks<true, MT == 1>(cb_lds);
        } else {
            if (all) run_chunks<false, true>(cb_lds);
            else run_chunks<false, MT == 1>(cb_lds);
        }
    }

    // The full chunks c0 .. cf - 1, D at a time, the next D loading while
    // one set computes (two register sets in turn, so no copies), then the
    // ragged last chunk of the row (Kin % 64 != 0).
    template <bool kG16, bool kAll>
    __device__ __forceinline__ void run_chunks(const float* cb_lds)
    {
        const int c0 = c0_, c1 = c1_, cf = cf_;
        const int n16 = P.Kin >> 4;
        if (c0 < cf) {
            XChunk<XT> xc;
            if (kXPre) xc.load(xsrc, (int64_t)c0 * TQ_CHUNK);
            Slot<K, LAYOUT> nxt[D];
            auto run = [&](int c, const Slot<K, LAYOUT> (&set)[D]) {
#pragma unroll
                for (int j = 0; j < D; ++j) {
                    if (c + j < cf) {
                        XChunk<XT> xn;
                        if (kXPre && c + j + 1 < cf) xn.load(xsrc, (int64_t)(c + j + 1) * TQ_CHUNK);
                        compute<true, kG16, kAll>(c + j, 4, set[j], &xc, cb_lds);
                        if (kXPre) xc = xn;
                    }
                }
            };
            for (int c = c0;; c += 2 * D) {
#pragma unroll
                for (int j = 0; j < D; ++j) load_slot(c + D + j, nxt[j]);
                run(c, cur);
                if (c + D >= cf) break;
#pragma unroll
                for (int j = 0; j < D; ++j) load_slot(c + 2 * D + j, cur[j]);
                run(c + D, nxt);
                if (c + 2 * D >= cf) break;
            }
        }
        if (cf < c1) {
            Slot<K, LAYOUT> s;
            load_slot(cf, s);
            compute<false, kG16, kAll>(cf, n16 - 4 * cf, s, nullptr, cb_lds);
        }
    }
};

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t quant4(f32x4 v, float inv)
{
    // per element: rne(fl(x * inv)) clamped to [-127, 127] -- the steps of tq_act_quant_int8
    const float e[4] = {v.x, v.y, v.z, v.w};
    uint32_t b = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float r = rintf(__fmul_rn(e[j], inv));
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        b |= ((uint32_t)(uint8_t)(int8_t)(int)r) << (8 * j);
    }
    return b;
}

// Per-token absmax int8 quantisation of the problem's activations into LDS,
// by every thread of the workgroup (the same operations as tq_act_quant_int8).
__device__ __forceinline__ void quantize_to_lds(const tq_prob_dev& P, uint32_t* xq, float* sx, float* wmax)
{
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int n4 = P.Kin >> 2;
    constexpr int kHeld = TQ_Q8_HELD;    // 16-byte vectors a thread keeps in registers
    for (int m = 0; m < P.M; ++m) {
        const GLOBAL_AS f32x4* xr = (const GLOBAL_AS f32x4*)((const float*)P.x + (int64_t)m * P.Kin);
        const bool held = kHeld > 0 && n4 <= kHeld * nthr;
        f32x4 v[kHeld > 0 ? kHeld : 1];
        float a = 0.0f;
        if (held) {
#pragma unroll
            for (int j = 0; j < kHeld; ++j) {
                const int i = tid + j * nthr;
                v[j] = i < n4 ? xr[i] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
#pragma unroll
            for (int j = 0; j < kHeld; ++j)
                a = fmaxf(a, fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w))));
        } else {
            for (int i = tid; i < n4; i += nthr) {
                const f32x4 u = xr[i];
                a = fmaxf(a, fmaxf(fmaxf(fabsf(u.x), fabsf(u.y)), fmaxf(fabsf(u.z), fabsf(u.w))));
            }
        }
        a = wave_max(a);
        if ((tid & 63) == 0) wmax[tid >> 6] = a;
        __syncthreads();
        a = wmax[0];
        for (int w = 1; w < (nthr >> 6); ++w) a = fmaxf(a, wmax[w]);
        const float inv = a > 0.0f ? 127.0f / a : 0.0f;
        uint32_t* row = xq + (m * P.Kin >> 2);
        if (held) {
#pragma unroll
            for (int j = 0; j < kHeld; ++j) {
                const int i = tid + j * nthr;
                if (i < n4) row[i] = quant4(v[j], inv);
            }
        } else {
            for (int i = tid; i < n4; i += nthr) row[i] = quant4(xr[i], inv);
        }
        if (tid == 0) sx[m] = a > 0.0f ? a / 127.0f : 0.0f;
        __syncthreads();
    }
}

// Row block `rb` of one problem; this wave is column split `wave` of `nwaves`.
// `red` is the row block's own LDS area for the partial sums.  Every wave of
// the workgroup calls this once (inactive waves with active = false) because
// it contains a workgroup barrier.
template <int XT, int LAYOUT, int K, int MT>
__device__ __forceinline__ void rowblock(const tq_prob_dev& P, const int rb, const int wave,
                                         const int nwaves, uint32_t* red, const float* cb_lds,
                                         const void* xsrc, float* sx_lds, const bool active,
                                         void* q8_lds, float* wmax_lds, const uint8_t* lut)
{
    float* sx_lds_w = sx_lds;
    constexpr bool kInt = XT == TQ_I8 || XT == TQ_F32_Q8;
    using A = typename AccT<XT>::type;
    constexpr bool kGroup = LAYOUT != TQ_SCALE_TENSOR;
    const int lane = threadIdx.x & 63;
    const int NC = P.NC;
    const int g = P.g;
    const int M = P.M;
    const int cpu = (!kGroup || g <= 64) ? 1 : (g >> 6);
    const int nunits = (NC + cpu - 1) / cpu;
    const int c0 = active ? ((nunits * wave) / nwaves) * cpu : 0;
    const int c1 = active ? std::min(((nunits * (wave + 1)) / nwaves) * cpu, NC) : 0;

    RowBlock<XT, LAYOUT, K, MT> blk(P, rb, xsrc, lut);
    if (XT == TQ_F32_Q8 && !TQ_Q8_EARLY_LOADS) quantize_to_lds(P, (uint32_t*)q8_lds, sx_lds_w, wmax_lds);
    blk.begin(c0, c1);
    if (XT == TQ_F32_Q8 && TQ_Q8_EARLY_LOADS) {
        // the first chunks are in flight while the workgroup quantises the activations
        quantize_to_lds(P, (uint32_t*)q8_lds, sx_lds_w, wmax_lds);
    }
    blk.finish(cb_lds);
    auto& p = blk.p;
    auto& out = blk.out;

    // Partial sums to LDS; wave 0 adds them in wave order and writes y.
    constexpr int R = kGroup ? MT : MT * K;
    if (nwaves > 1) {
        if (wave > 0) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                if (kGroup) {
                    red[((wave * R) + m) * 64 + lane] = __float_as_uint(out[m]);
                } else {
#pragma unroll
                    for (int k = 0; k < K; ++k) {
                        const A v = p[m][k];
                        red[((wave * R) + m * K + k) * 64 + lane] =
                            kInt ? (uint32_t)(int)v : __float_as_uint((float)v);
                    }
                }
            }
        }
        __syncthreads();
        if (wave != 0 || !active) return;   // split 0 of an active block finishes it
        for (int wv = 1; wv < nwaves; ++wv) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                if (kGroup) {
                    out[m] += __uint_as_float(red[((wv * R) + m) * 64 + lane]);
                } else {
#pragma unroll
                    for (int k = 0; k < K; ++k) {
                        const uint32_t bits = red[((wv * R) + m * K + k) * 64 + lane];
                        if (kInt) p[m][k] += (A)(int)bits;
                        else p[m][k] += (A)__uint_as_float(bits);
                    }
                }
            }
        }
    }

    const int64_t n = (int64_t)rb * TQ_ROWS + lane;
    if (!active || n >= P.N) return;
    float ts[K];
    if (!kGroup) {
#pragma unroll
        for (int k = 0; k < K; ++k) ts[k] = ld_uniform(reinterpret_cast<const float*>(P.scales) + k);
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        if (m >= M) break;
        float yv;
        if (kInt) {
            const float xs = XT == TQ_F32_Q8 ? sx_lds[m] : ld_uniform(P.x_scale + m);
            if (!kGroup && K == 1) {
                // bit exact: y = fl(float(acc) * fl(s_w * s_x))
                const float cm = __fmul_rn(ts[0], xs);
                yv = __fmul_rn((float)p[m][0], cm);
                if (P.acc) ((GLOBAL_AS int32_t*)P.acc)[(int64_t)m * P.N + n] = (int)p[m][0];
            } else if (!kGroup) {
                float t = 0.0f;
#pragma unroll
                for (int k = 0; k < K; ++k) t = fmaf(ts[k], (float)p[m][k], t);
                yv = t * xs;
            } else {
                yv = out[m] * xs;
            }
        } else {
            if (!kGroup) {
                float t = 0.0f;
#pragma unroll
                for (int k = 0; k < K; ++k) t = fmaf(ts[k] * enc_scale<XT>(), (float)p[m][k], t);
                yv = t;
            } else {
                yv = out[m];
            }
        }
        ((GLOBAL_AS float*)P.y)[(int64_t)m * P.N + n] = yv;
    }
}

// One workgroup: `nrb` row blocks starting at rb0, each split over
// blockDim / (64 * nrb) waves.
template <int XT, int LAYOUT, int K, int MT>
__device__ __forceinline__ void gemv_body(const tq_prob_dev& P, int rb0, int nrb)
{
    extern __shared__ uint32_t tq_dyn[];     // [reduction areas][int8 activations]
    __shared__ float cb_lds[TQ_CB_SLOTS];
    __shared__ float sx_lds[TQ_MAX_M_GEMV];
    __shared__ float wmax[16];
    using B3T = B3Table<MT == 1 ? 16 : 8>;
    __shared__ __attribute__((aligned(16))) uint8_t lut[LAYOUT == TQ_SCALE_CODEBOOK_B3 ? B3T::kBytes
                                                        : (XT == TQ_BF16 ? kLutBytes : 16)];
    constexpr bool kGroup = LAYOUT != TQ_SCALE_TENSOR;
    constexpr int Rw = kGroup ? MT : MT * K;          // partial sums per lane
    constexpr bool kCb = LAYOUT == TQ_SCALE_CODEBOOK || LAYOUT == TQ_SCALE_CODEBOOK_B3;
    if (kCb && threadIdx.x < TQ_CB_SLOTS) cb_lds[threadIdx.x] = f16_to_f32(P.cb[threadIdx.x]);
    if constexpr (LAYOUT == TQ_SCALE_CODEBOOK_B3) B3T::fill(lut);
    else if constexpr (XT == TQ_BF16) fill_bf16_lut(lut);
    if (kCb || XT == TQ_BF16) __syncthreads();
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int nwaves = (int)(blockDim.x >> 6);
    const int S = nwaves / nrb;                       // waves per row block
    const int r = wave / S, split = wave - r * S;
    const int rb = rb0 + r;
    const bool active = rb * TQ_ROWS < P.N;
    const void* xsrc = P.x;
    uint32_t* xq = nullptr;
    if (XT == TQ_F32_Q8) {
        const int red_words = S > 1 ? nwaves * Rw * 64 : 0;
        xq = tq_dyn + red_words;
        xsrc = xq;     // filled inside rowblock, after its first loads are issued
    }
    rowblock<XT, LAYOUT, K, MT>(P, rb, split, S, tq_dyn + r * S * Rw * 64, cb_lds, xsrc, sx_lds, active,
                                xq, wmax, lut);
}

template <int XT, int LAYOUT, int K, int MT>
__global__ __launch_bounds__(1024) void k_gemv_single(tq_prob_dev P)
{
    gemv_body<XT, LAYOUT, K, MT>(P, (int)blockIdx.x, 1);
}

// A whole stack in one launch: workgroup i takes item i, `nrb` row blocks of
// one problem (items are ordered longest first by the host).
template <int XT, int LAYOUT, int K, int MT>
__global__ __launch_bounds__(1024) void k_gemv_grouped(const tq_prob_dev* __restrict__ probs,
                                                       const int2* __restrict__ items, int nrb)
{
    const int2 it = ld_uniform_struct(items + blockIdx.x);
    if (it.x < 0) return;    // a hole the host left in the item list
    const tq_prob_dev P = ld_uniform_struct(probs + it.x);
    gemv_body<XT, LAYOUT, K, MT>(P, it.y, nrb);
}

// One item per wave, for bf16 activations: wave w of workgroup b takes item
// b * waves + w, one 64-row block of one problem (the host keeps the token
// slices of one row block in one workgroup).  The workgroup's waves share
// the trit table, as in the grouped kernel, but each wave has its own
// problem.  No column split, no codebook: the only workgroup barrier is the
// table fill.
template <int XT, int LAYOUT, int K, int MT>
__global__ __launch_bounds__(1024) void k_gemv_wave_items(const tq_prob_dev* __restrict__ probs,
                                                                           const int2* __restrict__ items)
{
    static_assert(XT == TQ_BF16 && LAYOUT != TQ_SCALE_CODEBOOK && LAYOUT != TQ_SCALE_CODEBOOK_B3,
                  "per-wave items: bf16, no codebook");
    __shared__ float cb_lds[1];
    __shared__ float sx_lds[1];
    __shared__ __attribute__((aligned(16))) uint8_t lut[kLutBytes];
    fill_bf16_lut(lut);
    __syncthreads();
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int2 it = ld_uniform_struct(items + (int64_t)blockIdx.x * (blockDim.x >> 6) + wave);
    if (it.x < 0) return;    // a hole the host left in the item list
    const tq_prob_dev P = ld_uniform_struct(probs + it.x);
    rowblock<XT, LAYOUT, K, MT>(P, it.y, 0, 1, nullptr, cb_lds, P.x, sx_lds, it.y * TQ_ROWS < P.N, nullptr,
                                nullptr, lut);
}

}  // namespace tqk

namespace tqk {

typedef void (*single_fn)(tq_prob_dev);
typedef void (*grouped_fn)(const tq_prob_dev*, const int2*, int);
typedef void (*wave_items_fn)(const tq_prob_dev*, const int2*);

// tokens per pass of each M tier (more tokens are taken in slices of the last)
constexpr int kTiers = 2;
constexpr int kMT[kTiers] = {1, TQ_PASS_TOKENS};
// family = ((x_type * 4 + layout) * 4 + (K - 1)) * kTiers + M tier; 32 families per x_type.
// CODEBOOK_B3 (three digits combined into one value) is kernel K = 1, bf16 only.
constexpr int kLayouts = 4;
constexpr int kPerXT = 4 * kLayouts * kTiers;
constexpr int kXTypes = 4;

template <int XT, int LAYOUT, int K>
constexpr bool decode_exists() { return LAYOUT != TQ_SCALE_CODEBOOK_B3 || (XT == TQ_BF16 && K == 1); }

// The per-wave item kernel where the host uses it (bf16, several tokens per
// pass, no codebook), else none.
template <int XT, int LAYOUT, int K, int MT>
constexpr wave_items_fn wave_items_of()
{
    if constexpr (MT == 1 || XT != TQ_BF16 || LAYOUT == TQ_SCALE_CODEBOOK || LAYOUT == TQ_SCALE_CODEBOOK_B3)
        return nullptr;
    else return &k_gemv_wave_items<XT, LAYOUT, K, MT>;
}
template <int XT, int LAYOUT, int K, int MT>
constexpr single_fn single_of_t()
{
    if constexpr (!decode_exists<XT, LAYOUT, K>()) return nullptr;
    else return &k_gemv_single<XT, LAYOUT, K, MT>;
}
template <int XT, int LAYOUT, int K, int MT>
constexpr grouped_fn grouped_of_t()
{
    if constexpr (!decode_exists<XT, LAYOUT, K>()) return nullptr;
    else return &k_gemv_grouped<XT, LAYOUT, K, MT>;
}

// families of one (x_type, M tier): index = layout * 4 + (K - 1)
template <int F>
struct FamOf {
    static constexpr int K = F % 4 + 1;
    static constexpr int layout = F / 4;
};

template <int XT, int MT, int... Fs>
struct TablesXT {
    static constexpr single_fn single[] = {single_of_t<XT, FamOf<Fs>::layout, FamOf<Fs>::K, MT>()...};
    static constexpr grouped_fn grouped[] = {grouped_of_t<XT, FamOf<Fs>::layout, FamOf<Fs>::K, MT>()...};
    static constexpr wave_items_fn wave[] = {wave_items_of<XT, FamOf<Fs>::layout, FamOf<Fs>::K, MT>()...};
};

template <int XT, int MT, int... Is>
constexpr auto make_tables(std::integer_sequence<int, Is...>) { return TablesXT<XT, MT, Is...>{}; }

template <int XT, int MT>
using TablesFor = decltype(make_tables<XT, MT>(std::make_integer_sequence<int, 4 * kLayouts>{}));

// one translation unit per (x_type, M tier) defines its pair of tables
const single_fn* single_table(int x_type, int mti);
const grouped_fn* grouped_table(int x_type, int mti);
#define TQ_DECLARE_TABLES(xt, mti) \
    const single_fn* single_table_##xt##_##mti(); const grouped_fn* grouped_table_##xt##_##mti();
TQ_DECLARE_TABLES(0, 0) TQ_DECLARE_TABLES(0, 1)
TQ_DECLARE_TABLES(1, 0) TQ_DECLARE_TABLES(1, 1)
TQ_DECLARE_TABLES(2, 0) TQ_DECLARE_TABLES(2, 1)
TQ_DECLARE_TABLES(3, 0) TQ_DECLARE_TABLES(3, 1)
// per-wave item kernels of the 4-token tier (bf16 activations)
const wave_items_fn* wave_table_1_1();

}  // namespace tqk
