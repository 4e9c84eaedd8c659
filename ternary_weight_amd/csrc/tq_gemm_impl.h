#pragma once
// libtq: prefill kernels (any M) on the matrix cores -- tq_gemm and
// tq_gemm_grouped.
//
// What is computed is the definition in tq.h.  With many tokens the product
// is a dense contraction X[M][Kin] . T_k[N][Kin]^T per plane, so it runs on
// MFMA: the trits are decoded to the MFMA operand type in registers (int8 or
// bf16 values in {-1, 0, +1}; no weight multiply ever reaches the result
// beyond +-1), a partial sum per plane and group is accumulated by the matrix
// core (int32 exactly for int8 activations, fp32 for bf16), and the group's
// scale is applied once when the group ends (sasori page, "K and g"); a
// per-tensor scale is applied once at the very end (QORA-LLM-2B page,
// "Ternary GEMV (No Multiplication)").
//
// Mapping onto CDNA4.  A workgroup is 2 x 2 waves; a wave owns FM x FN tiles
// of 16 x 16 outputs (16 FM tokens by 16 FN weight rows).  Per step a wave
// loads, for each token tile, 16 bytes per lane of x (row = lane % 16, the
// lane group q = lane / 16 takes one quarter of the step's columns) and, for
// each weight tile, one dword of codes per lane: in the blob (tq_layout.h) a
// dword is 16 consecutive columns of one row, exactly the quarter-step of the
// int8 MFMA v_mfma_i32_16x16x64_i8 (64 columns per step), or a half dword for
// the bf16 MFMA v_mfma_f32_16x16x32_bf16 (32 columns per step).  Each decoded
// weight tile is reused by the FM token tiles, each token tile by the FN
// weight tiles.  x is read straight from global memory (the workgroup's other
// waves and neighbouring workgroups hit it in L1/L2); there is no LDS.
//
// Result tile layout of a 16 x 16 MFMA: lane l holds column l % 16 (a weight
// row n) of rows 4 (l / 16) + e, e = 0..3 (tokens m).
#include "tq_internal.h"
#include "tq_decode.h"

namespace tqm {

using namespace tqk;

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;   // 2 x 2 waves

template <int XT>
struct Mfma;

template <>
struct Mfma<TQ_I8> {
    static constexpr int kStep = 64;        // columns per MFMA
    using Part = i32x4;
    static __device__ __forceinline__ Part run(u32x4 a, u32x4 b, Part c)
    {
        return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b),
                                                     c, 0, 0, 0);
    }
    // int8 trits of the lane's 16 columns: the whole dword
    static __device__ __forceinline__ u32x4 decode(uint32_t w, int /*half*/)
    {
        uint32_t t[4];
        decode_i8(w, t);
        return u32x4{t[0], t[1], t[2], t[3]};
    }
    // the decoded trits are exactly +-1
    static constexpr float kScale = 1.0f;
};

// Two bf16 values {0, +2, -2} from the codes in bytes `b` and `b + 1` of a
// field-extracted dword f (one 2-bit code per byte): the first v_perm_b32
// moves the two codes to bytes 1 and 3 with zero bytes between, the second
// looks each up in a 4-byte table (0x00, 0x40, 0xC0, 0x00: the high bytes of
// bf16 0, 2, -2, 0; the low bytes of these values are zero).
template <int b>
__device__ __forceinline__ uint32_t bf16_pair(uint32_t f)
{
    constexpr uint32_t sel = 0x000C000Cu | ((uint32_t)b << 8) | ((uint32_t)(b + 1) << 24);
    const uint32_t s = __builtin_amdgcn_perm(0u, f, sel);
    return __builtin_amdgcn_perm(0u, 0x00C04000u, s);
}

template <>
struct Mfma<TQ_BF16> {
    static constexpr int kStep = 32;
    using Part = f32x4;
    static __device__ __forceinline__ Part run(u32x4 a, u32x4 b, Part c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    }
    // bf16 trits (times 2) of 8 consecutive columns: half `half` of the dword
    // (columns 8 half .. 8 half + 7 = fields 2 half and 2 half + 1)
    static __device__ __forceinline__ u32x4 decode(uint32_t w, int half)
    {
        const uint32_t lo = (w >> (4 * half)) & 0x03030303u;        // columns 8h + b
        const uint32_t hi = (w >> (4 * half + 2)) & 0x03030303u;    // columns 8h + 4 + b
        return u32x4{bf16_pair<0>(lo), bf16_pair<2>(lo), bf16_pair<0>(hi), bf16_pair<2>(hi)};
    }
    static constexpr float kScale = 0.5f;   // undo the factor 2 of the decoded values
};

// One workgroup tile (32 FM tokens x 32 FN weight rows) of one problem.
template <int XT, int LAYOUT, int K, int FM, int FN>
__device__ __forceinline__ void gemm_tile(const tq_prob_dev& P, int tm, int tn)
{
    using MF = Mfma<XT>;
    using Part = typename MF::Part;
    constexpr int KS = MF::kStep;
    constexpr int ESZ = XT == TQ_I8 ? 1 : 2;             // bytes per activation
    constexpr int QCOLS = KS / 4;                         // columns per lane group
    // int8, one plane, per-tensor scale: the int32 sum is the result
    constexpr bool kDirect = XT == TQ_I8 && LAYOUT == TQ_SCALE_TENSOR && K == 1;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, q = lane >> 4;
    const int M = P.M, N = P.N, Kin = P.Kin, NC = P.NC;
    const int NB = (N + 63) >> 6;
    const int m0 = tm * (32 * FM) + (wave & 1) * (16 * FM);
    const int n0 = tn * (32 * FN) + (wave >> 1) * (16 * FN);

    // x rows of the lane (rows past M repeat row M - 1; their results are not stored)
    const uint8_t* xrow[FM];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int row = min(m0 + 16 * fm + r, M - 1);
        xrow[fm] = (const uint8_t*)P.x + ((int64_t)row * Kin + q * QCOLS) * ESZ;
    }
    // code slots of the lane's weight rows (rows past the last block read block 0; not stored)
    const uint8_t* crow[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        const int n = n0 + 16 * fn + r;
        const int rb = n >> 6;
        crow[fn] = P.codes + (rb < NB ? ((int64_t)rb * NC * K * 64 + (n & 63)) * 16 : 0);
    }

    // Steps: segment (group, or the whole row for a per-tensor scale), then
    // plane, then the segment's MFMA steps.
    const int nks = (Kin + KS - 1) / KS;                       // MFMA steps per row
    const int seg_steps = LAYOUT == TQ_SCALE_TENSOR ? nks : P.g / KS;
    const int nseg = LAYOUT == TQ_SCALE_TENSOR ? 1 : Kin / P.g;
    const int total = nseg * K * seg_steps;

    Part part[FM][FN];
    f32x4 acc[kDirect ? 1 : FM][kDirect ? 1 : FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            part[fm][fn] = Part{0, 0, 0, 0};
            if (!kDirect) acc[kDirect ? 0 : fm][kDirect ? 0 : fn] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    auto load = [&](int seg, int k, int j, u32x4 (&a)[FM], uint32_t (&w)[FN]) {
        const int ks = seg * seg_steps + j;                     // MFMA step along the row
        const int col = ks * KS;
        const bool in = col + q * QCOLS < Kin;                  // Kin % 16 == 0: all or nothing
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            a[fm] = in ? *(const GLOBAL_AS u32x4*)(xrow[fm] + (int64_t)col * ESZ) : u32x4{0u, 0u, 0u, 0u};
        const int c = XT == TQ_I8 ? ks : ks >> 1;               // 64-column chunk
        const int dw = XT == TQ_I8 ? q : 2 * (ks & 1) + (q >> 1);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
            w[fn] = *(const GLOBAL_AS uint32_t*)(crow[fn] + ((int64_t)c * K + k) * 1024 + dw * 4);
    };

    u32x4 a_nxt[FM];
    uint32_t w_nxt[FN];
    int seg = 0, k = 0, j = 0;
    load(0, 0, 0, a_nxt, w_nxt);
    for (int t = 0; t < total; ++t) {
        u32x4 a[FM];
        uint32_t w[FN];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) a[fm] = a_nxt[fm];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) w[fn] = w_nxt[fn];
        const int cseg = seg, ck = k, cj = j;
        if (++j == seg_steps) {
            j = 0;
            if (++k == K) {
                k = 0;
                ++seg;
            }
        }
        if (t + 1 < total) load(seg, k, j, a_nxt, w_nxt);

        // scales of this (segment, plane) for the lane's weight rows
        float sc[FN];
        if (!kDirect && cj == seg_steps - 1) {
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                if (LAYOUT == TQ_SCALE_TENSOR) {
                    sc[fn] = ld_uniform(((const float*)P.scales) + ck) * MF::kScale;
                } else {
                    const int n = n0 + 16 * fn + r;
                    const int rb = min(n >> 6, NB - 1);
                    const uint32_t word = *(const GLOBAL_AS uint32_t*)(P.scales +
                        ((((int64_t)rb * P.NGD + (cseg >> 1)) * K + ck) * 64 + (n & 63)) * 4);
                    sc[fn] = f16_to_f32((cseg & 1) ? (word >> 16) : (word & 0xFFFFu)) * MF::kScale;
                }
            }
        }

        const int half = XT == TQ_I8 ? 0 : (q & 1);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const u32x4 b = MF::decode(w[fn], half);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) part[fm][fn] = MF::run(a[fm], b, part[fm][fn]);
        }

        if (!kDirect && cj == seg_steps - 1) {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[kDirect ? 0 : fm][kDirect ? 0 : fn][e] =
                            fmaf(sc[fn], (float)part[fm][fn][e], acc[kDirect ? 0 : fm][kDirect ? 0 : fn][e]);
                    part[fm][fn] = Part{0, 0, 0, 0};
                }
        }
    }

    // epilogue: lane holds weight row n = n0 + 16 fn + r of tokens m0 + 16 fm + 4 q + e
    float sw = 0.0f;
    if (kDirect) sw = ld_uniform((const float*)P.scales);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = m0 + 16 * fm + 4 * q + e;
            if (m >= M) continue;
            float xs = 1.0f;
            if (XT == TQ_I8) xs = P.x_scale[m];
            const float cm = kDirect ? sw * xs : xs;   // fl32(s_w * x_scale[m]), one rounding
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int n = n0 + 16 * fn + r;
                if (n >= N) continue;
                const int64_t o = (int64_t)m * N + n;
                if (kDirect) {
                    const int v = part[fm][fn][e];
                    P.y[o] = (float)v * cm;
                    if (P.acc) P.acc[o] = v;
                } else {
                    P.y[o] = XT == TQ_I8 ? acc[kDirect ? 0 : fm][kDirect ? 0 : fn][e] * cm
                                         : acc[kDirect ? 0 : fm][kDirect ? 0 : fn][e];
                }
            }
        }
    }
}

template <int XT, int LAYOUT, int K, int FM, int FN>
__global__ __launch_bounds__(kThreads) void k_gemm_single(tq_prob_dev P, int tiles_m)
{
    const int tile = blockIdx.x;
    gemm_tile<XT, LAYOUT, K, FM, FN>(P, tile % tiles_m, tile / tiles_m);
}

// Grouped: item i = (problem, tile); tiles of a problem run token-tile fastest.
template <int XT, int LAYOUT, int K, int FM, int FN>
__global__ __launch_bounds__(kThreads) void k_gemm_grouped(const tq_prob_dev* probs, const int2* items)
{
    const int2 it = items[blockIdx.x];
    const tq_prob_dev P = ld_uniform_struct(probs + it.x);
    const int tiles_m = (P.M + 32 * FM - 1) / (32 * FM);
    gemm_tile<XT, LAYOUT, K, FM, FN>(P, it.y % tiles_m, it.y / tiles_m);
}

}  // namespace tqm
