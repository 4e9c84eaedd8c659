#pragma once
// libtq: matrix-core product for a few bf16 tokens (M <= 16) -- the kernels
// behind tq_gemv's and the grouped plans' several-token bf16 path, and
// tq_gemm with at most 16 tokens.
//
// What is computed is the definition in tq.h (sasori page, "K and g": the
// sum over planes and groups of a scale times the group's trit-weighted sum
// of x; d3 card, "Quantization details": the codec's three digits weigh 9,
// 3 and 1 and a group's scale is its codebook entry).
//
// Mapping onto CDNA4.  A workgroup is 4 waves; wave w owns the 64-row block
// 4 tile + w (the wide kernels, for int8 with one plane and a per-tensor
// scale and 8 or more tokens: the two blocks 2 (4 tile + w) and the next,
// with the same x fragments) and one MFMA tile of 16 tokens (rows past M
// read zeros).  The
// wave walks its block one 64-column chunk at a time, every plane of the
// chunk in one step:
//   - lane l loads row l's 16-byte slot of each plane (one coalesced 1 KiB
//     load per plane; tq_layout.h), the scale words of its row that the
//     chunk's groups need, and its x fragments of the chunk (token l % 16);
//   - the slots and scale words go through an LDS stage of the wave's own
//     (double buffered; only the wave touches it and its LDS accesses
//     complete in order, so no barrier), from which lane (r, q) reads the
//     code dwords of its MFMA fragments: row 16 fn + r of tile fn;
//   - per plane and chunk, 2 steps of v_mfma_f32_16x16x32_bf16 (groups of 32
//     and more, per-tensor scale) or 4 of v_mfma_f32_16x16x16_bf16 (groups
//     of 16, the codec), 4 MFMAs each (tiles fn = 0..3), into a partial sum
//     per plane and tile; a group's scales are applied once when it ends;
//   - the codec's three two-bit digit planes are combined per column into
//     one operand of exact values 9 d0 + 3 d1 + d2 (a 64-entry table of bf16
//     values in LDS), so a group takes one MFMA and one codebook scale per
//     tile, not one per plane.
// Loads run NBUF - 1 chunks ahead.  The per-chunk bookkeeping (offsets, the
// chunk's groups) is a few scalar instructions per chunk, where a kernel
// stepping one MFMA step of one plane at a time spends them on every step.
//
// The codes decode to bf16 {0, +2, -2} (the factor 2 is taken out with the
// scale); the compact base-3 codes through the pair-code table in LDS, as
// bf16 pairs of the combined digit values (exact integers in [-13, 13]).
#include <type_traits>

#include "tq_gemm_impl.h"

namespace tqm {

#ifndef TQ_SKINNY_NBUF
#define TQ_SKINNY_NBUF 4   // chunks in flight (even: the stage parity follows the buffer index)
#endif
// The codec's combined-digit kernel: two chunks in flight at three waves per
// SIMD (136 VGPRs; Llama-8B-shaped codec stack, 16 tokens: 1.53 ms, against
// 1.58 ms with four chunks at two waves per SIMD and 1.60 ms with six; four
// chunks at three waves per SIMD spill).
#ifndef TQ_SKINNY_COMB_NBUF
#define TQ_SKINNY_COMB_NBUF 2
#endif
#define TQ_SKINNY_COMB_NBUF_OR(comb, other) ((comb) ? TQ_SKINNY_COMB_NBUF : (other))

// The two-bit decode of these kernels.  One field of a code dword (one
// 2-bit code per byte: columns 4p .. 4p + 3, tq_layout.h) gives four bf16
// values {0, +2, -2} with one lookup of their high bytes (a v_perm_b32 whose
// selectors are the codes; the low bytes of the values are zero), then the
// odd and the even columns as two bf16 pairs: (4p + 1, 4p + 3) and (4p,
// 4p + 2).  19 vector instructions per 16 columns, against 23 for pairs of
// consecutive columns.  The MFMA's k order within a lane is free, so the x
// fragment is permuted to the same order, once per step for every plane and
// tile (xodd_even).
__device__ __forceinline__ u32x2 bf16_odd_even(uint32_t f)
{
    const uint32_t hi = __builtin_amdgcn_perm(0u, 0x00C04000u, f);   // high bytes of columns 0..3
    return u32x2{hi & 0xFF00FF00u,                                    // columns 1, 3
                 __builtin_amdgcn_perm(0u, hi, 0x020C000Cu)};         // columns 0, 2
}
// 32-column steps: half h of the dword (fields 2h and 2h + 1), columns
// 8h + (1, 3), (0, 2), (5, 7), (4, 6)
__device__ __forceinline__ u32x4 decode_oe32(uint32_t w, int h)
{
    const u32x2 lo = bf16_odd_even((w >> (4 * h)) & 0x03030303u);
    const u32x2 hi = bf16_odd_even((w >> (4 * h + 2)) & 0x03030303u);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
}
// 16-column steps: field p, columns 4p + (1, 3), (0, 2)
__device__ __forceinline__ u32x2 decode_oe16(uint32_t w, int p)
{
    return bf16_odd_even((w >> (2 * p)) & 0x03030303u);
}
// x (bf16, consecutive columns) in the same order: from dwords (c, c + 1),
// (c + 2, c + 3) the pairs (c + 1, c + 3) and (c, c + 2)
template <typename F>
__device__ __forceinline__ F xodd_even(F x)
{
    F y;
#pragma unroll
    for (int i = 0; i < (int)(sizeof(F) / 4); i += 2) {
        y[i] = __builtin_amdgcn_perm(x[i + 1], x[i], 0x07060302u);
        y[i + 1] = __builtin_amdgcn_perm(x[i + 1], x[i], 0x05040100u);
    }
    return y;
}

// How a group ends: never (per-tensor scale: at the end of the row), after
// every MFMA step (groups of the step's width: each step's MFMAs start from
// zero), or after g / KS steps (larger groups: the sums are cleared when the
// group's scales have been applied).
enum { kGroupNone = 0, kGroupStep = 1, kGroupSteps = 2 };

// Dwords of a wave's stage: a row's code dwords (4 per plane; the compact
// codes' 10 padded to 12), their stride an odd multiple of 4 dwords so that
// the 16 rows of a fragment read fall in distinct banks, then the row's
// scale words of the chunk (GROUP_F16: one pair word per plane, two for
// groups of 16; the codec: the two index words that hold the chunk's four
// groups; TENSOR: none).
template <int LAYOUT, int K, int KS>
struct SkinnyStage {
    static constexpr bool kB3 = LAYOUT == TQ_SCALE_CODEBOOK_B3;
    static constexpr int CDS = kB3 ? 12 : (K % 2 ? 4 * K : 4 * K + 4);
    static constexpr int SWN = LAYOUT == TQ_SCALE_TENSOR
                                   ? 0
                                   : (LAYOUT == TQ_SCALE_CODEBOOK || kB3 ? 2 : (KS == 16 ? 2 * K : K));
    static constexpr int WST = 64 * (CDS + SWN);   // dwords per wave and stage
};

// The codec's two-bit digit planes combined into one operand per group
// (skinny_tile), and the table size that takes.
template <int XT, int LAYOUT, int K, int KS>
constexpr bool skinny_comb() { return XT == TQ_BF16 && LAYOUT == TQ_SCALE_CODEBOOK && K == 3 && KS == 16; }
// 64-row blocks per wave (RB): one, or two -- the "wide" kernels, for int8
// with one plane and a per-tensor scale and 8 or more tokens: the same x
// fragments serve both blocks, so a wave loads half as many x bytes per code
// byte (BitNet-2B-shaped stack, 16 tokens: 57.7 -> 60.7% of HBM, 8 tokens
// 64.6 -> 66.4%; 4 tokens the same, 2 tokens 77.8 -> 75.9%).
template <int XT, int LAYOUT, int K, int KS>
constexpr bool skinny_wide_ok() { return XT == TQ_I8 && LAYOUT == TQ_SCALE_TENSOR && K == 1; }
template <int XT, int LAYOUT, int K, int KS>
constexpr int skinny_lut_bytes()
{
    return skinny_comb<XT, LAYOUT, K, KS>() ? D3Table::kBytes : b3_lut_bytes<LAYOUT>();
}
// The codebook (and the table of the compact codes or of the combined digits) in LDS.
template <int XT, int LAYOUT, int K, int KS>
__device__ __forceinline__ void skinny_stage_tables(const tq_prob_dev& P, float* cb_lds, uint8_t* lut)
{
    if constexpr (skinny_comb<XT, LAYOUT, K, KS>()) {
        if (threadIdx.x < TQ_CB_SLOTS) cb_lds[threadIdx.x] = f16_to_f32(P.cb[threadIdx.x]);
        D3Table::fill(lut);
        __syncthreads();
    } else {
        stage_codebook<LAYOUT>(P, cb_lds, lut);
    }
}

template <int XT, int LAYOUT, int K, int KS, int GM, int RB>
__device__ __forceinline__ void skinny_tile(const tq_prob_dev& P, int tn, const LDS_AS float* cb_lds,
                                            const LDS_AS uint8_t* b3_lut, LDS_AS uint32_t* wlds)
{
    using MF = Mfma<XT, KS>;
    using Frag = typename MF::Frag;
    using Part = typename MF::Part;
    constexpr bool kI8 = XT == TQ_I8;
    constexpr int ESZ = kI8 ? 1 : 2;             // bytes per activation
    constexpr bool kB3 = LAYOUT == TQ_SCALE_CODEBOOK_B3;
    constexpr bool kCb = LAYOUT == TQ_SCALE_CODEBOOK || kB3;
    constexpr bool kTensor = LAYOUT == TQ_SCALE_TENSOR;
    // int8, one plane, per-tensor scale: the int32 sum is the result (exact)
    constexpr bool kDirect = kI8 && kTensor && K == 1;
    static_assert(!kB3 || (!kI8 && K == 1 && KS == 16), "compact base-3 codes: one stream, 16-column steps");
    static_assert(kI8 ? (KS == 64 && !kCb) : (KS == 32 || KS == 16), "MFMA step");
    static_assert((GM == kGroupNone) == kTensor, "group mode");
    // The codec's three two-bit digit planes (d = 3): each 16-column group's
    // digits are combined into one operand of exact values 9 d0 + 3 d1 + d2
    // through the combined-digit table, one MFMA and one codebook scale per
    // group and tile instead of one per plane.
    constexpr bool kComb = skinny_comb<XT, LAYOUT, K, KS>();
    constexpr int KP = kComb ? 1 : K;            // partial sums per tile: planes, or the one combined operand
    constexpr int KPC = 64 / KS;                 // MFMA steps per chunk
    using SS = SkinnyStage<LAYOUT, K, KS>;
    constexpr int NFN = 4 * RB;                           // 16-row tiles per wave
    static_assert(RB == 1 || (RB == 2 && skinny_wide_ok<XT, LAYOUT, K, KS>()), "two blocks per wave: int8, one plane");
    constexpr int CDS = SS::CDS, SWN = SS::SWN, WST = SS::WST * RB;
    // chunks in flight: four (Llama-8B-shaped K = 3 stack, 16 tokens: 1.23
    // against 1.28 ms with two; the compact codes 1.29 against 1.54 ms), two
    // where four would not fit the registers of two waves per SIMD, and two
    // for int8 with group scales (111 instead of 189 registers, four waves
    // per SIMD instead of two; routed experts, K = 3, 64 tokens: 4.37
    // against 4.46 ms) and for codebook scales on digit planes other than
    // the three the combined kernel takes (measured when the three-digit
    // codec still ran one plane at a time: 16 tokens 1.80 against 1.87 ms)
    constexpr int NBUF = (K == 4 || (XT == TQ_I8 && LAYOUT == TQ_SCALE_GROUP_F16) ||
                          (LAYOUT == TQ_SCALE_CODEBOOK && !kComb))
                             ? 2 : TQ_SKINNY_COMB_NBUF_OR(kComb, TQ_SKINNY_NBUF);
    static_assert(NBUF % 2 == 0 && NBUF >= 2, "chunks in flight");
    constexpr int XL = 64 / KS;                  // x loads per chunk (one MFMA step's fragment each)
    using XF = typename std::conditional<KS * ESZ == 64, u32x4, u32x2>::type;
    static_assert(sizeof(XF) == sizeof(Frag), "an x load is one MFMA step's fragment");
    constexpr int CL = kB3 ? 3 : K;              // code loads per chunk (a slot per plane; B3: three parts)
    using B3T = B3Table<8>;   // pair-code table, 8 copies (32 KiB)

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, q = lane >> 4;
    const int M = P.M, N = P.N, Kin = P.Kin, NC = P.NC;
    const int NB = (N + 63) >> 6;
    const int rb = (tn * 4 + wave) * RB;          // the wave's first row block
    const int n0 = rb * 64;

    // Buffer resources (tq_decode.h): a lane whose VGPR offset is at or past
    // the size reads zeros, so token rows past M and row blocks past N read
    // zeros; the per-chunk SGPR offsets stay inside the data.
    const __amdgpu_buffer_rsrc_t rx = rsrc(P.x, (int64_t)M * Kin * ESZ);
    const __amdgpu_buffer_rsrc_t rc =
        rsrc(P.codes, kB3 ? (int64_t)NB * NC * TQ_B3_CHUNK_BYTES : (int64_t)NB * NC * K * 1024);
    const __amdgpu_buffer_rsrc_t rs = rsrc(P.scales, kTensor ? 256 : (kCb ? (int64_t)NB * P.NID * 256
                                                                          : (int64_t)NB * P.NGD * K * 256));
    // x: lane (r, q) takes token r, in step s columns s KS + q KS / 4 .. + KS / 4 - 1
    const uint32_t xv0 = ((uint32_t)r * (uint32_t)Kin + (uint32_t)q * (KS / 4)) * ESZ;
    // codes: lane l loads row n0 + l; the block's offset is in the VGPR offset
    const uint32_t cv = kB3 ? (uint32_t)rb * (uint32_t)NC * TQ_B3_CHUNK_BYTES + (uint32_t)lane * 16u
                            : ((uint32_t)rb * (uint32_t)NC * K * 64u + (uint32_t)lane) * 16u;
    const uint32_t cv2 = kB3 ? (uint32_t)rb * (uint32_t)NC * TQ_B3_CHUNK_BYTES + 2048u + (uint32_t)lane * 8u : 0u;
    const uint32_t sv = kTensor ? 0u
                                : (kCb ? ((uint32_t)rb * (uint32_t)P.NID * 64u + (uint32_t)lane) * 4u
                                       : ((uint32_t)rb * (uint32_t)P.NGD * K * 64u + (uint32_t)lane) * 4u);
    // log2 g, and MFMA steps per group
    const int lg = kTensor ? 0 : 31 - __builtin_clz((unsigned)P.g);
    const int spg = kTensor ? 1 : P.g / KS;

    // the wave's two stages: row l's code dwords at l CDS, then its scale
    // words at 64 CDS + 64 j + l
    LDS_AS uint32_t* const st0 = wlds + wave * WST;
    LDS_AS uint32_t* const st1 = wlds + (4 + wave) * WST;

    // B3: lane (r, q)'s 20 bits of step s (columns 4q .. 4q + 3 of the
    // group) start at bit 80 s + 20 q of its row's stream: dword i, shift h
    uint32_t b3_i[KPC], b3_h[KPC];
#pragma unroll
    for (int s = 0; s < KPC; ++s) {
        const uint32_t bit = 80u * s + 20u * (uint32_t)q;
        b3_i[s] = bit >> 5;
        b3_h[s] = bit & 31u;
    }
    const uint32_t b3_copy = kB3 ? B3T::copy_offset() : 0u;
    // kComb: rotations that bring field q (bits 2q, 2q + 1 of every byte) of
    // plane k to bits 2k + 1, 2k + 2, so that each byte becomes 2 g, the
    // byte offset of its column's combined value in the table
    const uint32_t rot0 = (2u * (uint32_t)q - 1u) & 31u, rot1 = (2u * (uint32_t)q - 3u) & 31u,
                   rot2 = (2u * (uint32_t)q - 5u) & 31u;
    // kComb: the code dwords of the chunk, row 16 fn + r, plane k (read once per chunk)
    u32x4 cwv[kComb ? 4 : 1][kComb ? 3 : 1];

    u32x4 cbuf[NBUF][CL * RB];                    // B3: parts 0, 1 and (low half) 2; block-major
    uint32_t sbuf[NBUF][SWN > 0 ? SWN : 1];
    XF xbuf[NBUF][XL];

    // the scale words of chunk c, whose groups are (64 c) / g onwards:
    // GROUP_F16 with groups of 32 and more, the pair word (gd, k) at
    // (gd K + k) 256 of the chunk's groups, gd = (64 c / g) / 2, per plane;
    // groups of 16, pair words 2c and 2c + 1 per plane; the codec, the index
    // word of the chunk's first group and the next
    auto scale_soff = [&](int c) -> uint32_t {
        if constexpr (kCb) return (uint32_t)(((c << 6) >> lg) / 6) * 256u;
        else if constexpr (KS == 16) return (uint32_t)(2 * c) * K * 256u;
        else return (uint32_t)(((c << 6) >> lg) >> 1) * K * 256u;
    };
    auto load = [&](int c, u32x4 (&cb)[CL * RB], uint32_t (&sw)[SWN > 0 ? SWN : 1], XF (&xa)[XL]) {
        c = c < NC ? c : NC - 1;   // a prefetch past the last chunk loads the last again (never used)
        const uint32_t xv = xv0 + (uint32_t)c * (64u * ESZ);
#pragma unroll
        for (int i = 0; i < XL; ++i) xa[i] = buffer_load<XF>(rx, xv + (uint32_t)i * (KS * ESZ), 0);
        if constexpr (kB3) {
            const uint32_t so = (uint32_t)c * TQ_B3_CHUNK_BYTES;
            cb[0] = buffer_load<u32x4, kCacheNT>(rc, cv, so);
            cb[1] = buffer_load<u32x4, kCacheNT>(rc, cv + 1024u, so);
            const u32x2 t = buffer_load<u32x2, kCacheNT>(rc, cv2, so);
            cb[2] = u32x4{t[0], t[1], 0u, 0u};
        } else {
            const uint32_t so = (uint32_t)c * K * 1024u;
#pragma unroll
            for (int b = 0; b < RB; ++b)
#pragma unroll
                for (int k = 0; k < CL; ++k)
                    cb[b * CL + k] = buffer_load<u32x4, kCacheNT>(
                        rc, cv + (uint32_t)b * (uint32_t)NC * K * 1024u + (uint32_t)k * 1024u, so);
        }
        if constexpr (SWN > 0) {
            const uint32_t so = scale_soff(c);
#pragma unroll
            for (int j = 0; j < SWN; ++j) sw[j] = buffer_load<uint32_t>(rs, sv + (uint32_t)j * 256u, so);
        }
    };
    auto stage_write = [&](LDS_AS uint32_t* st, const u32x4 (&cb)[CL * RB], const uint32_t (&sw)[SWN > 0 ? SWN : 1]) {
        LDS_AS uint32_t* row = st + lane * CDS;
        if constexpr (kB3) {
            *(LDS_AS u32x4*)(row) = cb[0];
            *(LDS_AS u32x4*)(row + 4) = cb[1];
            *(LDS_AS u32x2*)(row + 8) = u32x2{cb[2][0], cb[2][1]};
        } else {
#pragma unroll
            for (int b = 0; b < RB; ++b)
#pragma unroll
                for (int k = 0; k < CL; ++k) *(LDS_AS u32x4*)(row + 64 * CDS * b + 4 * k) = cb[b * CL + k];
        }
#pragma unroll
        for (int j = 0; j < SWN; ++j) st[64 * CDS + 64 * j + lane] = sw[j];
    };

    Part part[KP][NFN];
    f32x4 acc[NFN];
#pragma unroll
    for (int fn = 0; fn < NFN; ++fn) {
        acc[fn] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KP; ++k) part[k][fn] = Part{0, 0, 0, 0};
    }

    // the weight fragment of plane k, tile fn, step s from the stage
    auto frag = [&](const LDS_AS uint32_t* st, int k, int fn, int s) -> Frag {
        const LDS_AS uint32_t* row = st + (16 * fn + r) * CDS;
        if constexpr (kI8) {
            // the one step: dword q of the plane's slot, int8 trits of its 16 columns in order
            return MF::decode(row[4 * k + q], q);
        } else if constexpr (kB3) {
            const uint32_t i = b3_i[s];
            const uint32_t wv = __builtin_amdgcn_alignbit(row[i + 1], row[i], b3_h[s]);
            const uint32_t a0 = ((wv & 0x3FFu) << B3T::kShift) | b3_copy;
            const uint32_t a1 = (((wv >> 10) & 0x3FFu) << B3T::kShift) | b3_copy;
            Frag f;
            f[0] = *(const LDS_AS uint32_t*)(b3_lut + a0);
            f[1] = *(const LDS_AS uint32_t*)(b3_lut + a1);
            return f;
        } else if constexpr (kComb) {
            // step s: dword s of each plane's slot, field q: the lane's four
            // columns' codes as table offsets 2 g, one per byte; then the
            // pairs (1, 3) and (0, 2) (the odd-even order of x)
            const uint32_t g = (__builtin_amdgcn_alignbit(cwv[fn][2][s], cwv[fn][2][s], rot2) & 0x60606060u) |
                               (__builtin_amdgcn_alignbit(cwv[fn][1][s], cwv[fn][1][s], rot1) & 0x18181818u) |
                               (__builtin_amdgcn_alignbit(cwv[fn][0][s], cwv[fn][0][s], rot0) & 0x06060606u);
            const LDS_AS uint16_t* t = (const LDS_AS uint16_t*)b3_lut;
            typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
            u16x2 p13, p02;
            p13[0] = *(const LDS_AS uint16_t*)((const LDS_AS uint8_t*)t + __builtin_amdgcn_ubfe(g, 8, 8));
            p13[1] = *(const LDS_AS uint16_t*)((const LDS_AS uint8_t*)t + (g >> 24));
            p02[0] = *(const LDS_AS uint16_t*)((const LDS_AS uint8_t*)t + (g & 0xFFu));
            p02[1] = *(const LDS_AS uint16_t*)((const LDS_AS uint8_t*)t + __builtin_amdgcn_ubfe(g, 16, 8));
            Frag f;
            f[0] = __builtin_bit_cast(uint32_t, p13);
            f[1] = __builtin_bit_cast(uint32_t, p02);
            return f;
        } else if constexpr (KS == 32) {
            // step s: dword 2 s + q / 2 of the plane's slot, half q % 2
            return decode_oe32(row[4 * k + 2 * s + (q >> 1)], q & 1);
        } else {
            // step s: dword s, field q
            return decode_oe16(row[4 * k + s], q);
        }
    };
    // the codec: the chunk's two index words of tile fn's row, read once per
    // chunk (idxw), and the index of the chunk's first group in the first
    uint32_t idxw[kCb ? 4 : 1][2];
    int idx0 = 0;
    auto read_idx = [&](const LDS_AS uint32_t* st, int c) {
        if constexpr (kCb) {
            const int g0 = (c << 6) >> lg;                        // the chunk's first group
            idx0 = g0 - 6 * (g0 / 6);
#pragma unroll
            for (int fn = 0; fn < 4; ++fn) {
                idxw[fn][0] = st[64 * CDS + 16 * fn + r];
                idxw[fn][1] = st[64 * CDS + 64 + 16 * fn + r];
            }
        }
    };
    // the scale of plane k of group `grp` (a global group index), for tile
    // fn's row, from the stage's scale words of the chunk
    auto group_scale = [&](const LDS_AS uint32_t* st, int c, int grp, int k, int fn) -> float {
        const LDS_AS uint32_t* sw = st + 64 * CDS + 16 * fn + r;
        if constexpr (kCb) {
            const int j = idx0 + grp - ((c << 6) >> lg);         // 0 .. 7: word j / 6, field j % 6
            const uint32_t w = j >= 6 ? idxw[fn][1] : idxw[fn][0];
            const float cb = cb_lds[(w >> (5 * (j >= 6 ? j - 6 : j))) & 31u];
            if constexpr (kB3 || kComb) {
                return cb;                                         // the table holds the combined values
            } else {
                float wgt = MF::kScale;                            // digit plane k weighs 3^(K - 1 - k)
#pragma unroll
                for (int i = 1; i < K; ++i)
                    if (i < K - k) wgt *= 3.0f;
                return cb * wgt;
            }
        } else {
            // GROUP_F16: the pair word of group grp for plane k
            int word;
            if constexpr (KS == 16) word = ((grp >> 1) - 2 * c) * K + k;   // words 2c and 2c + 1
            else word = k;                                                // the chunk's word of the plane
            const uint32_t w = sw[64 * word];
            return f16_to_f32((grp & 1) ? (w >> 16) : (w & 0xFFFFu)) * MF::kScale;
        }
    };
    auto apply = [&](const LDS_AS uint32_t* st, int c, int grp) {
#pragma unroll
        for (int fn = 0; fn < NFN; ++fn)
#pragma unroll
            for (int k = 0; k < KP; ++k) {
                const float sc = group_scale(st, c, grp, k, fn);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[fn][e] = fmaf(sc, (float)part[k][fn][e], acc[fn][e]);
            }
    };
    // x columns past Kin (a ragged last step of a per-tensor scale): zero,
    // so that whatever the next token's row holds there adds nothing
    auto mask_x = [&](int c, XF (&xa)[XL]) {
        if constexpr (kI8) return;   // integer products: zero trits add exactly zero
#pragma unroll
        for (int i = 0; i < XL; ++i)
#pragma unroll
            for (int d = 0; d < (int)(sizeof(XF) / 4); ++d) {
                const int col = 64 * c + i * KS + q * (KS / 4) + 2 * d;
                const uint32_t keep = col + 1 < Kin ? 0xFFFFFFFFu : (col < Kin ? 0x0000FFFFu : 0u);
                xa[i][d] &= keep;
            }
    };

    // chunk c from the stage st with x fragments xa: its valid steps, the
    // groups that end in it
    const int nks = (Kin + KS - 1) / KS;          // MFMA steps in a row
    auto compute = [&](int c, const LDS_AS uint32_t* st, XF (&xa)[XL]) {
        const int nv = nks - c * KPC;              // valid steps of the chunk (>= 1; more than KPC: all)
        if (kTensor && c == NC - 1 && Kin % KS != 0) mask_x(c, xa);
        read_idx(st, c);
        if constexpr (kComb) {
#pragma unroll
            for (int fn = 0; fn < NFN; ++fn)
#pragma unroll
                for (int k = 0; k < 3; ++k) cwv[fn][k] = *(const LDS_AS u32x4*)(st + (16 * fn + r) * CDS + 4 * k);
        }
        auto one_step = [&](int s, bool zero) {
            // x in the weight fragments' column order (the compact codes'
            // table gives consecutive columns)
            const Frag a = __builtin_bit_cast(Frag, kB3 || kI8 ? xa[s] : xodd_even(xa[s]));
#pragma unroll
            for (int k = 0; k < KP; ++k)
#pragma unroll
                for (int fn = 0; fn < NFN; ++fn) {
                    const Frag b = frag(st, k, fn, s);
                    part[k][fn] = MF::run(a, b, zero ? Part{0, 0, 0, 0} : part[k][fn]);
                }
            if constexpr (GM == kGroupStep) apply(st, c, c * KPC + s);
        };
#pragma unroll
        for (int s = 0; s < KPC; ++s) {
            if (s > 0 && s >= nv) break;
            // a group of one step starts from zero in the MFMA itself
            one_step(s, GM == kGroupStep);
            if constexpr (GM == kGroupSteps) {
                // the group's last step: its scales, then the sums start
                // again (clearing them here keeps the MFMAs free of a
                // branch, which would keep every fragment of a step live)
                const int t = c * KPC + s;
                if (((t + 1) & (spg - 1)) == 0) {
                    apply(st, c, (t * KS) >> lg);
#pragma unroll
                    for (int k = 0; k < KP; ++k)
#pragma unroll
                        for (int fn = 0; fn < NFN; ++fn) part[k][fn] = Part{0, 0, 0, 0};
                }
            }
        }
    };

    // Chunk t lives in register buffer t % NBUF and stage t % 2.  One step:
    // the loads of chunk t + NBUF - 1, the stage write of chunk t + 1, the
    // MFMAs of chunk t.
    auto step = [&](int u, int t) {
        constexpr int kAhead = NBUF - 1;
        load(t + kAhead, cbuf[(u + kAhead) % NBUF], sbuf[(u + kAhead) % NBUF], xbuf[(u + kAhead) % NBUF]);
        __builtin_amdgcn_sched_barrier(0);   // keep the loads ahead of this chunk's work
        stage_write((u & 1) ? st0 : st1, cbuf[(u + 1) % NBUF], sbuf[(u + 1) % NBUF]);
        compute(t, (u & 1) ? st1 : st0, xbuf[u]);
    };
#pragma unroll
    for (int u = 0; u + 1 < NBUF; ++u) load(u, cbuf[u], sbuf[u], xbuf[u]);
    stage_write(st0, cbuf[0], sbuf[0]);
    int t = 0;
    for (; t + NBUF <= NC; t += NBUF) {
#pragma unroll
        for (int u = 0; u < NBUF; ++u) step(u, t + u);
    }
#pragma unroll
    for (int u = 0; u + 1 < NBUF; ++u) {   // the last NC % NBUF chunks, already loaded
        if (t + u < NC) step(u, t + u);
    }
    if constexpr (GM == kGroupNone && !kDirect) {
        // per-tensor scale: one fp32 per plane, after the whole row
#pragma unroll
        for (int k = 0; k < KP; ++k) {
            const float sc = ld_uniform(((const float*)P.scales) + k) * MF::kScale;
#pragma unroll
            for (int fn = 0; fn < NFN; ++fn)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[fn][e] = fmaf(sc, (float)part[k][fn][e], acc[fn][e]);
        }
    }

    // lane (r, q) holds weight row n0 + 16 fn + r of tokens 4 q + e; int8
    // activations take their token's scale (one plane with a per-tensor
    // scale: y = fl32(float(acc) * fl32(s_w * x_scale[m])), tq.h)
    const float s_w = kDirect ? ld_uniform((const float*)P.scales) : 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int m = 4 * q + e;
        if (m >= M) continue;
        const float xs = kI8 ? P.x_scale[m] : 1.0f;
        const float cm = kDirect ? s_w * xs : xs;
#pragma unroll
        for (int fn = 0; fn < NFN; ++fn) {
            const int n = n0 + 16 * fn + r;
            if (n >= N) continue;
            const int64_t o = (int64_t)m * N + n;
            if constexpr (kDirect) {
                const int v = part[0][fn][e];
                P.y[o] = (float)v * cm;
                if (P.acc) P.acc[o] = v;
            } else {
                P.y[o] = kI8 ? acc[fn][e] * cm : acc[fn][e];
            }
        }
    }
}

// The group mode of a launch: groups of the step's width end with every
// step, larger ones after g / KS steps (one kernel takes both; the branch is
// uniform).
template <int XT, int LAYOUT, int K, int KS, int RB>
__device__ __forceinline__ void skinny_dispatch(const tq_prob_dev& P, int tn, const LDS_AS float* cb_lds,
                                                const LDS_AS uint8_t* b3_lut, LDS_AS uint32_t* wlds)
{
    if constexpr (LAYOUT == TQ_SCALE_TENSOR) {
        skinny_tile<XT, LAYOUT, K, KS, kGroupNone, RB>(P, tn, cb_lds, b3_lut, wlds);
    } else {
        if (P.g == KS) skinny_tile<XT, LAYOUT, K, KS, kGroupStep, RB>(P, tn, cb_lds, b3_lut, wlds);
        else skinny_tile<XT, LAYOUT, K, KS, kGroupSteps, RB>(P, tn, cb_lds, b3_lut, wlds);
    }
}

#ifndef TQ_SKINNY_COMB_WPS
#define TQ_SKINNY_COMB_WPS 3
#endif
// Waves per SIMD the register budget is sized for.
template <int XT, int LAYOUT, int K, int KS>
constexpr int skinny_waves() { return skinny_comb<XT, LAYOUT, K, KS>() ? TQ_SKINNY_COMB_WPS : 2; }

// The kernels' body: the tables, then the tile of 64 RB rows per wave.
template <int XT, int LAYOUT, int K, int KS, int RB>
__device__ __forceinline__ void skinny_body(const tq_prob_dev& P, int tn)
{
    __shared__ float cb_lds[TQ_CB_SLOTS];
    __shared__ __attribute__((aligned(16))) uint8_t b3_lut[skinny_lut_bytes<XT, LAYOUT, K, KS>()];
    __shared__ __attribute__((aligned(16))) uint32_t wlds[8 * SkinnyStage<LAYOUT, K, KS>::WST * RB];
    skinny_stage_tables<XT, LAYOUT, K, KS>(P, cb_lds, b3_lut);
    skinny_dispatch<XT, LAYOUT, K, KS, RB>(P, tn, (const LDS_AS float*)cb_lds, (const LDS_AS uint8_t*)b3_lut,
                                           (LDS_AS uint32_t*)wlds);
}

template <int XT, int LAYOUT, int K, int KS>
__global__ __launch_bounds__(kThreads, (skinny_waves<XT, LAYOUT, K, KS>())) void k_gemm_skinny(tq_prob_dev P, int /*tiles_m*/)
{
    skinny_body<XT, LAYOUT, K, KS, 1>(P, blockIdx.x);
}

// Grouped: item i = (problem, tile); one token tile per problem.
template <int XT, int LAYOUT, int K, int KS>
__global__ __launch_bounds__(kThreads, (skinny_waves<XT, LAYOUT, K, KS>())) void k_gemm_skinny_grouped(const tq_prob_dev* probs, const int2* items)
{
    const int2 it = items[blockIdx.x];
    const tq_prob_dev P = ld_uniform_struct(probs + it.x);
    skinny_body<XT, LAYOUT, K, KS, 1>(P, it.y);
}

// Two 64-row blocks per wave (skinny_wide_ok).
template <int XT, int LAYOUT, int K, int KS>
__global__ __launch_bounds__(kThreads, 2) void k_gemm_skinny_wide(tq_prob_dev P, int /*tiles_m*/)
{
    skinny_body<XT, LAYOUT, K, KS, 2>(P, blockIdx.x);
}

template <int XT, int LAYOUT, int K, int KS>
__global__ __launch_bounds__(kThreads, 2) void k_gemm_skinny_wide_grouped(const tq_prob_dev* probs, const int2* items)
{
    const int2 it = items[blockIdx.x];
    const tq_prob_dev P = ld_uniform_struct(probs + it.x);
    skinny_body<XT, LAYOUT, K, KS, 2>(P, it.y);
}

}  // namespace tqm
