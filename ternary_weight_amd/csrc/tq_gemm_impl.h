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
// Mapping onto CDNA4.  A workgroup is 4 waves, 2 x 2 (tokens x weight rows)
// for prefill or 1 x 4 for a few tokens; a wave owns FM x FN tiles of
// 16 x 16 outputs (16 FM tokens by 16 FN weight rows).  An MFMA's operands
// are 16 rows by one step of columns, each lane holding row lane % 16 and
// the quarter q = lane / 16 of the step's columns: for x, 16 bytes; for the
// weights, one dword of codes (in the blob, tq_layout.h, a dword is 16
// consecutive columns of one row), exactly the quarter-step of the int8 MFMA
// v_mfma_i32_16x16x64_i8 (64 columns per step), or a half dword for the bf16
// MFMA v_mfma_f32_16x16x32_bf16 (32 columns per step), or a quarter dword for
// v_mfma_f32_16x16x16_bf16 (16 columns per step: one group of the d = 3
// codec, whose scale is applied after each step).  Each decoded weight tile
// is reused by the FM token tiles, each token tile by the FN weight tiles.
// In the 2 x 2 kernels the workgroup stages each step's x tile and code
// dwords in LDS once, and the waves read their fragments from there.
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

constexpr int kThreads = 256;   // 4 waves
#ifndef TQ_GEMM_NBUF
#define TQ_GEMM_NBUF 4             // steps in flight of the prefill kernels
#endif
#ifndef TQ_GEMM_PAIR
#define TQ_GEMM_PAIR 1             // two steps per barrier where the registers allow
#endif
#ifndef TQ_GEMM_B3_NBUF
#define TQ_GEMM_B3_NBUF 4          // steps in flight of the compact codec's kernels
#endif
#ifndef TQ_GEMM_WAVES_PER_SIMD
#define TQ_GEMM_WAVES_PER_SIMD 2   // register budget: two waves per SIMD, so that one
                                   // wave's trit decode overlaps the other's MFMAs
#endif

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Outputs of at most 1 GiB are stored through a buffer resource; kYPast is
// the offset of an output past M or N: at or above the resource's size even
// when added to a row or column offset that is itself in range.
constexpr int64_t kYLean = (int64_t)1 << 30;
constexpr uint32_t kYPast = 1u << 30;

// The MFMA of one step of KS columns for activation type XT: operand
// fragments (16 tokens or 16 weight rows by KS columns, KS / 4 columns per
// lane group), partial-sum type, and the decode of the lane's columns from
// its dword of codes.
template <int XT, int KS>
struct Mfma;

template <>
struct Mfma<TQ_I8, 64> {
    using Frag = u32x4;
    using Part = i32x4;
    static __device__ __forceinline__ Part run(Frag a, Frag b, Part c)
    {
        return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b),
                                                     c, 0, 0, 0);
    }
    // int8 trits of the lane's 16 columns: the whole dword
    static __device__ __forceinline__ Frag decode(uint32_t w, int /*q*/)
    {
        uint32_t t[4];
        decode_i8(w, t);
        return Frag{t[0], t[1], t[2], t[3]};
    }
    // lane group q reads dword q of the step's 64-column chunk
    static __device__ __forceinline__ int chunk(int ks) { return ks; }
    static __device__ __forceinline__ int dword_lane(int q) { return q; }
    static __device__ __forceinline__ int dword_step(int /*ks*/) { return 0; }
    static constexpr float kScale = 1.0f;   // the decoded trits are exactly +-1
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
struct Mfma<TQ_BF16, 32> {
    using Frag = u32x4;
    using Part = f32x4;
    static __device__ __forceinline__ Part run(Frag a, Frag b, Part c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    }
    // bf16 trits (times 2) of 8 consecutive columns: half q & 1 of the dword
    // (columns 8h .. 8h + 7 = fields 2h and 2h + 1)
    static __device__ __forceinline__ Frag decode(uint32_t w, int q)
    {
        const int half = q & 1;
        const uint32_t lo = (w >> (4 * half)) & 0x03030303u;        // columns 8h + b
        const uint32_t hi = (w >> (4 * half + 2)) & 0x03030303u;    // columns 8h + 4 + b
        return Frag{bf16_pair<0>(lo), bf16_pair<2>(lo), bf16_pair<0>(hi), bf16_pair<2>(hi)};
    }
    static __device__ __forceinline__ int chunk(int ks) { return ks >> 1; }
    static __device__ __forceinline__ int dword_lane(int q) { return q >> 1; }
    static __device__ __forceinline__ int dword_step(int ks) { return 2 * (ks & 1); }
    static constexpr float kScale = 0.5f;   // undo the factor 2 of the decoded values
};

// 16 columns per step: one dword of codes, lane group q taking field q
// (columns 4q .. 4q + 3).  A step is exactly one group of 16, the group size
// of the d = 3 codec.
template <>
struct Mfma<TQ_BF16, 16> {
    using Frag = u32x2;
    using Part = f32x4;
    static __device__ __forceinline__ Part run(Frag a, Frag b, Part c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b),
                                                         c, 0, 0, 0);
    }
    static __device__ __forceinline__ Frag decode(uint32_t w, int q)
    {
        const uint32_t f = (w >> (2 * q)) & 0x03030303u;            // columns 4q + b
        return Frag{bf16_pair<0>(f), bf16_pair<2>(f)};
    }
    static __device__ __forceinline__ int chunk(int ks) { return ks >> 2; }
    static __device__ __forceinline__ int dword_lane(int /*q*/) { return 0; }
    static __device__ __forceinline__ int dword_step(int ks) { return ks & 3; }
    static constexpr float kScale = 0.5f;
};

template <typename F>
__device__ __forceinline__ F zero_frag()
{
    F z;
#pragma unroll
    for (int i = 0; i < (int)(sizeof(F) / 4); ++i) z[i] = 0u;
    return z;
}

// One workgroup tile of one problem: WM x (4 / WM) waves, each with FM x FN
// tiles of 16 x 16, so 16 FM WM tokens by 16 FN (4 / WM) weight rows.
// Loads through buffer resources: a 32-bit per-lane offset plus a uniform
// offset per step, no address arithmetic in the loop, and lanes whose offset
// is past the resource's size read zero (rows past M, row blocks past N).
// The host keeps every operand of a launch below 4 GiB.
// Position in the step sequence: segment (a group, or the whole row for a
// per-tensor scale), then plane, then the segment's MFMA steps.
// The codec's three two-bit digit planes combined into one operand per
// 16-column group (gemm_tile), and the table that takes.
template <int XT, int LAYOUT, int K, int KS>
constexpr bool gemm_comb() { return XT == TQ_BF16 && LAYOUT == TQ_SCALE_CODEBOOK && K == 3 && KS == 16; }

struct Cursor {
    int seg, k, j;
    __device__ __forceinline__ void advance(int seg_steps, int K)
    {
        if (++j == seg_steps) {
            j = 0;
            if (++k == K) {
                k = 0;
                ++seg;
            }
        }
    }
};

template <int XT, int LAYOUT, int K, int FM, int FN, int KS, int WM>
__device__ __forceinline__ void gemm_tile(const tq_prob_dev& P, int tm, int tn, const LDS_AS float* cb_lds,
                                          const LDS_AS uint8_t* b3_lut)
{
    using MF = Mfma<XT, KS>;
    using Part = typename MF::Part;
    using Frag = typename MF::Frag;
    constexpr int ESZ = XT == TQ_I8 ? 1 : 2;             // bytes per activation
    constexpr int QCOLS = KS / 4;                         // columns per lane group
    // int8, one plane, per-tensor scale: the int32 sum is the result
    constexpr bool kDirect = XT == TQ_I8 && LAYOUT == TQ_SCALE_TENSOR && K == 1;
    // the scale word of a (segment, plane) block: two f16 group scales, or six 5-bit codebook indices
    constexpr bool kWord = !kDirect && LAYOUT != TQ_SCALE_TENSOR;
    // x through LDS: the 2 x 2 kernels whose step is 64 bytes of a row (int8,
    // or 32 bf16 columns).  The workgroup loads its 16 FM WM rows once per
    // step, 16 bytes per thread and chunk, and every wave reads its fragments
    // from there instead of loading them again.
    constexpr int TM = 16 * FM * WM;
    constexpr bool kLds = WM == 2 && KS * ESZ == 64 && TM * 4 % kThreads == 0;
    constexpr int XCH = kLds ? TM * 4 / kThreads : 1;     // 16-byte chunks per thread and step
    // Two steps per barrier (the int8 one-plane kernel, whose registers allow
    // six steps in flight): the workgroup stage is a ring of NBUF steps, and
    // at every other step the waves meet once and stage the two steps after
    // the next.  Otherwise one barrier per step and a double-buffered stage.
    constexpr bool kPair = kLds && kDirect && TQ_GEMM_PAIR;
    // steps in flight (loads issued NBUF - 1 steps ahead)
    constexpr int NBUF = kPair ? 6 : LAYOUT == TQ_SCALE_CODEBOOK_B3 ? TQ_GEMM_B3_NBUF : TQ_GEMM_NBUF;
    constexpr int NST = kPair ? NBUF : 2;                  // stages of the workgroup's LDS ring
    // The codes go through LDS as well: the workgroup's TN rows' code dwords
    // of a step are CW per row (the whole 16-byte slot for int8, half of it
    // for bf16), loaded CPT consecutive dwords per thread.  Read in the MFMA
    // fragment layout straight from global memory, 16 lanes of a load would
    // sit 16 bytes apart, which costs the L1 about one access per two lanes.
    constexpr int TN = 16 * FN * (4 / WM);
    constexpr int CW = kLds ? (XT == TQ_I8 ? 4 : 2) : 1;
    constexpr int CPT = kLds ? TN * CW / kThreads : 1;
    static_assert(!kLds || ((CPT == 1 || CPT == 2 || CPT == 4) && CW % CPT == 0), "code dwords per thread");
    // Codes through a stage of the wave's own: the bf16 kernels without the
    // workgroup stage (the one-tile kernels, and 16-column steps), whose wave
    // owns one whole 64-row block.  Lane l loads row l's code dwords of the
    // step (half or a quarter of the row's 16 bytes) and its scale word, so
    // one load walks the block's 1 KiB slot in row order; the MFMA fragments
    // are read back from LDS.
    // Only the wave touches its stage, and a wave's LDS accesses complete in
    // order, so no barrier is needed.
    constexpr bool kWave = !kLds && XT == TQ_BF16 && FN == 4;
    // The codec's compact base-3 codes (CODEBOOK_B3): one combined value per
    // weight (K = 1 here), 16-column steps of 80 bits per row -- dwords
    // (5 d) / 2 .. + 2 of the 64-column chunk's ten, d = step % 4 -- staged
    // per wave, and decoded through the pair-code table: one MFMA and one
    // codebook scale per 16-column group, in place of one per digit plane.
    constexpr bool kB3 = LAYOUT == TQ_SCALE_CODEBOOK_B3;
    constexpr bool kCb = LAYOUT == TQ_SCALE_CODEBOOK || kB3;
    static_assert(!kB3 || (kWave && K == 1 && KS == 16), "compact base-3 codes: the per-wave stage, 16-column steps");
    // The codec's three two-bit digit planes: a step stages the group's
    // dword of each plane, and each column's three digits become one operand
    // of exact values 9 d0 + 3 d1 + d2 (the combined-digit table): one MFMA
    // and one codebook scale per group, as for the compact codes.
    constexpr bool kComb = gemm_comb<XT, LAYOUT, K, KS>();
    static_assert(!kComb || kWave, "combined digits: the per-wave stage");
    constexpr int KC = kComb ? 1 : K;                     // planes the steps walk (the combined operand: one)
    constexpr int CWW = kB3 || kComb ? 3 : KS / 16;       // code dwords of a row per step
    constexpr int WST = 64 * CWW + (kWord ? 64 : 0) + (kB3 ? 4 : 0);   // dwords per wave and stage (B3: a
                                                                      // pad dword read past the last row)

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, q = lane >> 4;
    const int M = P.M, N = P.N, Kin = P.Kin, NC = P.NC;
    const int NB = (N + 63) >> 6;
    static_assert(WM == 1 || WM == 2, "waves along the tokens");
    const int m0 = tm * (16 * FM * WM) + (wave % WM) * (16 * FM);
    const int n0 = tn * (16 * FN * (4 / WM)) + (wave / WM) * (16 * FN);

    const int64_t xbytes = (int64_t)M * Kin * ESZ;
    const __amdgpu_buffer_rsrc_t rc = rsrc(P.codes, kB3 ? (int64_t)NB * NC * TQ_B3_CHUNK_BYTES : (int64_t)NB * NC * K * 1024);
    const __amdgpu_buffer_rsrc_t rs = rsrc(P.scales, kCb ? (int64_t)NB * P.NID * 256 : (int64_t)NB * P.NGD * K * 256);
    uint32_t xoff[FM], coff[FN], soff[FN], cwoff = 0, swoff = 0;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) xoff[fm] = ((uint32_t)(m0 + 16 * fm + r) * Kin + q * QCOLS) * ESZ;
    // LDS staging: chunk id = thread + 256 i holds row id / 4, 16-byte column
    // chunk id % 4; a row's four chunks are stored XOR-swizzled by (row / 2) % 4,
    // so that the 8 lanes of one 128-byte LDS pass (32 banks of 4 bytes), rows
    // R .. R + 7 of one chunk, fall in distinct banks, for reads and writes
    uint32_t xoffl[XCH], xlds_w[XCH];
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
        const uint32_t id = threadIdx.x + kThreads * i, R = id >> 2, c = id & 3;
        xoffl[i] = ((uint32_t)(tm * TM + R) * Kin) * ESZ + 16 * c;
        xlds_w[i] = R * 64 + 16 * (c ^ ((R >> 1) & 3));
    }
    uint32_t xlds_r[FM];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const uint32_t R = (wave % WM) * (16 * FM) + 16 * fm + r;
        xlds_r[fm] = R * 64 + 16 * (q ^ ((R >> 1) & 3));
    }
    __shared__ __attribute__((aligned(16))) uint8_t xlds[kLds ? NST : 1][kLds ? TM * 64 : 16];
    // code stage: row R's dword d at R * CW + ((d + rot(R)) % CW), the int8
    // rotation rot = 2 ((R / 8) % 2) putting the 32 lanes of one LDS pass
    // (rows R .. R + 15, two dwords each) in distinct banks
    __shared__ __attribute__((aligned(16))) uint32_t clds[kLds ? NST : 1][kLds ? TN * CW : 4];
    uint32_t ccoff = 0, clds_w = 0, clds_w2 = 0, clds_r[FN];
    {
        const uint32_t T = threadIdx.x, R = T * CPT / CW, d0 = T * CPT % CW;
        const uint32_t n = tn * TN + R;
        const uint32_t rot = CW == 4 ? 2 * ((R >> 3) & 1) : 0;
        ccoff = ((n >> 6) * NC * K * 64 + (n & 63)) * 16 + d0 * 4;
        clds_w = R * CW + ((d0 + rot) % CW);
        clds_w2 = R * CW + ((d0 + 2 + rot) % CW);   // CPT = 4: the row's second half
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const uint32_t Rr = (wave / WM) * (16 * FN) + 16 * fn + r;
            const uint32_t rotr = CW == 4 ? 2 * ((Rr >> 3) & 1) : 0;
            clds_r[fn] = Rr * CW + ((MF::dword_lane(q) + rotr) % CW);
        }
    }
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        const uint32_t n = n0 + 16 * fn + r;
        coff[fn] = ((n >> 6) * NC * K * 64 + (n & 63)) * 16 + MF::dword_lane(q) * 4;
        soff[fn] = kCb ? ((n >> 6) * P.NID * 64 + (n & 63)) * 4 : ((n >> 6) * P.NGD * K * 64 + (n & 63)) * 4;
    }
    uint32_t cwoff2 = 0;   // B3: the lane's offset in its block's third part (dwords 8, 9)
    if constexpr (kWave) {
        const uint32_t n = n0 + lane;                      // n0 is a multiple of 64
        if constexpr (kB3) {
            // the block offset goes in the lane's offset, so that a block past
            // N is past the resource's size and reads zeros
            cwoff = (n >> 6) * NC * TQ_B3_CHUNK_BYTES + (n & 63) * 16;
            cwoff2 = (n >> 6) * NC * TQ_B3_CHUNK_BYTES + 2048 + (n & 63) * 8;
        } else {
            cwoff = ((n >> 6) * NC * K * 64 + (n & 63)) * 16;
        }
        swoff = kCb ? ((n >> 6) * P.NID * 64 + (n & 63)) * 4 : ((n >> 6) * P.NGD * K * 64 + (n & 63)) * 4;
    }
    // B3: where lane (r, q)'s 20 bits (columns 4q .. 4q + 3 of the step) sit
    // in its row's three staged dwords -- bit 16 (d % 2) + 20 q
    uint32_t b3_lo[2] = {0, 0}, b3_sh[2] = {0, 0};
    if constexpr (kB3) {
#pragma unroll
        for (int par = 0; par < 2; ++par) {
            const uint32_t o = 16u * par + 20u * (uint32_t)q;
            b3_lo[par] = o >> 5;
            b3_sh[par] = o & 31u;
        }
    }
    using B3T = B3Table<8>;   // pair-code table, 8 copies (32 KiB: more workgroups per unit, measured)
    const uint32_t b3_copy = kB3 ? B3T::copy_offset() : 0u;
    // combined digits: plane k's rotation, field q to bits 2k + 1, 2k + 2
    const uint32_t crot[3] = {(2u * (uint32_t)q - 1u) & 31u, (2u * (uint32_t)q - 3u) & 31u,
                              (2u * (uint32_t)q - 5u) & 31u};
    __shared__ __attribute__((aligned(16))) uint32_t wlds[kWave ? 2 : 1][kWave ? 4 * WST : 4];
    LDS_AS uint32_t* const wst0 = (LDS_AS uint32_t*)wlds[0] + (kWave ? wave * WST : 0);
    LDS_AS uint32_t* const wst1 = (LDS_AS uint32_t*)wlds[kWave ? 1 : 0] + (kWave ? wave * WST : 0);

    const int nks = (Kin + KS - 1) / KS;                       // MFMA steps per row
    const int seg_steps = LAYOUT == TQ_SCALE_TENSOR ? nks : P.g / KS;
    const int nseg = LAYOUT == TQ_SCALE_TENSOR ? 1 : Kin / P.g;
    const int total = nseg * KC * seg_steps;

    Part part[FM][FN];
    f32x4 acc[kDirect ? 1 : FM][kDirect ? 1 : FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            part[fm][fn] = Part{0, 0, 0, 0};
            if (!kDirect) acc[kDirect ? 0 : fm][kDirect ? 0 : fn] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    // Columns of x past Kin in a ragged last step read the next row (or zero
    // past the end); the codes there are padding (zero trits), so they add 0.
    constexpr int AREG = kLds ? XCH : FM;                  // x registers per step buffer
    constexpr int WREG = kLds ? CPT : kWave ? CWW : FN;    // code registers per step buffer
    constexpr int SREG = kWave ? 1 : FN;                   // scale words per step buffer
    Frag abuf[NBUF][AREG];
    uint32_t wbuf[NBUF][WREG], swbuf[NBUF][SREG];
    auto load = [&](const Cursor& cur, Frag (&a)[AREG], uint32_t (&w)[WREG], uint32_t (&sw)[SREG]) {
        // a cursor past the last step (the prefetch runs ahead of the end)
        // loads the last step again: the data is in cache and never used
        const bool past = cur.seg >= nseg;
        const Cursor c{past ? nseg - 1 : cur.seg, past ? KC - 1 : cur.k, past ? seg_steps - 1 : cur.j};
        const int ks = c.seg * seg_steps + c.j;                 // MFMA step along the row
        const uint32_t xs = (uint32_t)ks * (KS * ESZ);
        // x through a window from the step's first column to the end of x, so
        // that the columns of a ragged last step past the last row read zeros
        const __amdgpu_buffer_rsrc_t rxs = rsrc((const uint8_t*)P.x + xs, xbytes - xs);
        if (kLds) {
#pragma unroll
            for (int i = 0; i < AREG; ++i) a[i] = buffer_load<Frag>(rxs, xoffl[i], 0);
        } else {
#pragma unroll
            for (int i = 0; i < AREG; ++i) a[i] = buffer_load<Frag>(rxs, xoff[i], 0);
        }
        const uint32_t cs = ((uint32_t)MF::chunk(ks) * K + c.k) * 1024 + MF::dword_step(ks) * 4;
        if constexpr (kLds) {
            if constexpr (CPT == 4) {
                const u32x4 v = buffer_load<u32x4>(rc, ccoff, cs);
#pragma unroll
                for (int i = 0; i < CPT; ++i) w[i] = v[i];
            } else if constexpr (CPT == 2) {
                const u32x2 v = buffer_load<u32x2>(rc, ccoff, cs);
                w[0] = v[0];
                w[CPT - 1] = v[1];
            } else {
                w[0] = buffer_load<uint32_t>(rc, ccoff, cs);
            }
        } else if constexpr (kB3) {
            // dwords D0 .. D0 + 2 of the step's chunk: 0..7 in the two 16-byte
            // parts (lane * 16), 8..9 in the third (lane * 8)
            const uint32_t chunk = (uint32_t)ks >> 2, d = (uint32_t)ks & 3u, D0 = (5u * d) >> 1;
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                const uint32_t D = D0 + i;
                const bool third = D >= 8;
                const uint32_t so = chunk * TQ_B3_CHUNK_BYTES + (third ? (D - 8) * 4 : (D >> 2) * 1024 + (D & 3) * 4);
                w[i] = buffer_load<uint32_t>(rc, third ? cwoff2 : cwoff, so);
            }
        } else if constexpr (kComb) {
            // the step's dword (16 columns) of each digit plane
#pragma unroll
            for (int i = 0; i < 3; ++i) w[i] = buffer_load<uint32_t>(rc, cwoff, cs + (uint32_t)i * 1024u);
        } else if constexpr (kWave) {
            if constexpr (CWW == 2) {
                const u32x2 v = buffer_load<u32x2>(rc, cwoff, cs);
                w[0] = v[0];
                w[CWW - 1] = v[1];
            } else {
                w[0] = buffer_load<uint32_t>(rc, cwoff, cs);
            }
        } else {
#pragma unroll
            for (int fn = 0; fn < WREG; ++fn) w[fn] = buffer_load<uint32_t>(rc, coff[fn], cs);
        }
        if (kWord) {   // the block's word, with every step (no branch around a load)
            const uint32_t ss = kCb ? (uint32_t)(c.seg / 6) * 256
                                                            : ((uint32_t)(c.seg >> 1) * K + c.k) * 256;
            if constexpr (kWave) {
                sw[0] = buffer_load<uint32_t>(rs, swoff, ss);
            } else {
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) sw[fn] = buffer_load<uint32_t>(rs, soff[fn], ss);
            }
        }
    };
    // the weight operand of one fragment: the codes' decode, or (B3) two
    // pair-code table reads for the lane's 20 bits -- columns 4q, 4q + 1 and
    // 4q + 2, 4q + 3, each a bf16 pair in column order
    auto decode = [&](uint32_t wv) -> Frag {
        if constexpr (kB3) {
            const uint32_t a0 = ((wv & 0x3FFu) << B3T::kShift) | b3_copy;
            const uint32_t a1 = (((wv >> 10) & 0x3FFu) << B3T::kShift) | b3_copy;
            Frag f;
            f[0] = *(const LDS_AS uint32_t*)(b3_lut + a0);
            f[1] = *(const LDS_AS uint32_t*)(b3_lut + a1);
            return f;
        } else if constexpr (kComb) {
            // wv: the lane's four columns' 6-bit codes as table offsets 2 g,
            // one per byte; pairs (0, 1) and (2, 3) in column order
            typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
            const LDS_AS uint8_t* t = b3_lut;
            u16x2 p01, p23;
            p01[0] = *(const LDS_AS uint16_t*)(t + (wv & 0xFFu));
            p01[1] = *(const LDS_AS uint16_t*)(t + __builtin_amdgcn_ubfe(wv, 8, 8));
            p23[0] = *(const LDS_AS uint16_t*)(t + __builtin_amdgcn_ubfe(wv, 16, 8));
            p23[1] = *(const LDS_AS uint16_t*)(t + (wv >> 24));
            Frag f;
            f[0] = __builtin_bit_cast(uint32_t, p01);
            f[1] = __builtin_bit_cast(uint32_t, p23);
            return f;
        } else {
            return MF::decode(wv, q);
        }
    };
    auto compute = [&](const Cursor& c, const Frag (&a)[FM], const uint32_t (&w)[FN], const uint32_t (&swr)[SREG],
                       const LDS_AS uint32_t* wst) {
        static_assert(sizeof(a) == FM * sizeof(Frag), "fragments");
        // the first step of a group starts its sums from zero in the MFMA
        // itself (no registers to clear when the previous group ends)
        if (!kDirect && c.j == 0) {
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const Frag b = decode(w[fn]);
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) part[fm][fn] = MF::run(a[fm], b, Part{0, 0, 0, 0});
            }
        } else {
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const Frag b = decode(w[fn]);
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) part[fm][fn] = MF::run(a[fm], b, part[fm][fn]);
            }
        }
        if (kDirect || c.j != seg_steps - 1) return;
        // the block's scale for the lane's weight rows, applied once
        uint32_t sw[FN];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) sw[fn] = kWave ? (kWord ? wst[64 * CWW + 16 * fn + r] : 0u) : swr[kWave ? 0 : fn];
        float sc[FN];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            if (LAYOUT == TQ_SCALE_TENSOR) {
                sc[fn] = ld_uniform(((const float*)P.scales) + c.k) * MF::kScale;
            } else if (kB3 || kComb) {
                // the table holds the combined values exactly: the group's scale alone
                sc[fn] = cb_lds[(sw[fn] >> (5 * (c.seg % 6))) & 31u];
            } else if (LAYOUT == TQ_SCALE_CODEBOOK) {
                // digit plane k weighs 3^(K-1-k); the group's scale is cb[idx[n][group]]
                const uint32_t idx = (sw[fn] >> (5 * (c.seg % 6))) & 31u;
                float wgt = 1.0f;
#pragma unroll
                for (int i = 1; i < K; ++i)
                    if (i < K - c.k) wgt *= 3.0f;
                sc[fn] = cb_lds[idx] * (wgt * MF::kScale);
            } else {
                sc[fn] = f16_to_f32((c.seg & 1) ? (sw[fn] >> 16) : (sw[fn] & 0xFFFFu)) * MF::kScale;
            }
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[kDirect ? 0 : fm][kDirect ? 0 : fn][e] =
                        fmaf(sc[fn], (float)part[fm][fn][e], acc[kDirect ? 0 : fm][kDirect ? 0 : fn][e]);
            }
    };

    // Step s lives in buffer s % NBUF; loads run NBUF - 1 steps ahead of the
    // MFMAs.  No load sits under a branch, so the compiler's wait counts see
    // exactly which loads a step needs.  Loads issued past the last step
    // repeat the last step's addresses and are never consumed.
    // LDS stage of a step (double buffered): write the thread's chunks, and
    // read a wave's fragments.  One barrier per step separates them: before
    // it every wave has written stage t % 2 and finished reading stage
    // (t + 1) % 2, which is written next.
    auto lds_write = [&](int stage, const Frag (&a)[AREG], const uint32_t (&w)[WREG]) {
#pragma unroll
        for (int i = 0; i < AREG; ++i) *(LDS_AS Frag*)((LDS_AS uint8_t*)xlds[stage] + xlds_w[i]) = a[i];
        if constexpr (CPT == 4) {
            // the row's four dwords, rotated: two halves at their rotated places
            *(LDS_AS u32x2*)((LDS_AS uint32_t*)clds[stage] + clds_w) = u32x2{w[0], w[1]};
            *(LDS_AS u32x2*)((LDS_AS uint32_t*)clds[stage] + clds_w2) = u32x2{w[2], w[CPT - 1]};
        } else if constexpr (CPT == 2) {
            *(LDS_AS u32x2*)((LDS_AS uint32_t*)clds[stage] + clds_w) = u32x2{w[0], w[CPT - 1]};
        } else {
            ((LDS_AS uint32_t*)clds[stage])[clds_w] = w[0];
        }
    };
    auto lds_read = [&](int stage, Frag (&a)[FM], uint32_t (&w)[FN]) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) a[fm] = *(const LDS_AS Frag*)((const LDS_AS uint8_t*)xlds[stage] + xlds_r[fm]);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) w[fn] = ((const LDS_AS uint32_t*)clds[stage])[clds_r[fn]];
    };
    auto barrier = [&]() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
    // the wave's own stage (double buffered like the workgroup one): lane l
    // writes row l's code dwords and scale word; the fragments are read back
    // in the MFMA layout, row 16 fn + r, the lane group's dword
    auto wave_write = [&](int stage, const uint32_t (&w)[WREG], const uint32_t (&sw)[SREG]) {
        if constexpr (kB3 || kComb) {
            LDS_AS uint32_t* st = stage ? wst1 : wst0;
#pragma unroll
            for (int i = 0; i < 3; ++i) st[3 * lane + i] = w[i];   // stride 3: no bank conflicts
            st[64 * CWW + lane] = sw[0];
        } else if constexpr (kWave) {
            LDS_AS uint32_t* st = stage ? wst1 : wst0;
            if constexpr (CWW == 2) {
                *(LDS_AS u32x2*)(st + 2 * lane) = u32x2{w[0], w[CWW - 1]};
            } else {
                st[lane] = w[0];
            }
            if constexpr (kWord) st[64 * CWW + lane] = sw[0];
        }
    };
    auto wave_read = [&](int stage, uint32_t (&w)[FN]) {
        if constexpr (kB3) {
            // the stage of step s is s % 2, and the step's 80 bits start at
            // bit 16 (s % 2) of its first staged dword: the lane's 20 bits
            const LDS_AS uint32_t* st = stage ? wst1 : wst0;
            const uint32_t lo = b3_lo[stage], sh = b3_sh[stage];
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const uint32_t base = (16 * fn + r) * 3 + lo;
                w[fn] = __builtin_amdgcn_alignbit(st[base + 1], st[base], sh);
            }
        } else if constexpr (kComb) {
            // row 16 fn + r's dword of each plane, field q (bits 2q, 2q + 1 of
            // every byte) of plane k rotated to bits 2k + 1, 2k + 2: each byte
            // becomes 2 g, the offset of its column's value in the table
            const LDS_AS uint32_t* st = stage ? wst1 : wst0;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const LDS_AS uint32_t* row = st + (16 * fn + r) * 3;
                w[fn] = (__builtin_amdgcn_alignbit(row[2], row[2], crot[2]) & 0x60606060u) |
                        (__builtin_amdgcn_alignbit(row[1], row[1], crot[1]) & 0x18181818u) |
                        (__builtin_amdgcn_alignbit(row[0], row[0], crot[0]) & 0x06060606u);
            }
        } else if constexpr (kWave) {
            const LDS_AS uint32_t* st = stage ? wst1 : wst0;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) w[fn] = st[(16 * fn + r) * CWW + MF::dword_lane(q)];
        }
    };
    // one step: the loads of step t + NBUF - 1, then (LDS path) the staging of
    // step t + 1, then the MFMAs of step t
    auto step = [&](int u, Cursor& ld, Cursor& cp, bool issue) {
        constexpr int kAhead = NBUF - 1;
        const int v = (u + kAhead) % NBUF;
        if (issue) {
            load(ld, abuf[v], wbuf[v], swbuf[v]);
            ld.advance(seg_steps, KC);
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the loads ahead of this step's MFMAs
        if constexpr (kLds) {
            Frag a[FM];
            uint32_t w[FN];
            if constexpr (kPair) {
                // even steps: stages u + 2 and u + 3 were last read at steps
                // u - 4 and u - 3, and stages u, u + 1 were written at step
                // u - 2, all before this barrier; their loads were issued at
                // steps u - 3 and u - 2
                if (u % 2 == 0) {
                    barrier();
                    lds_write((u + 2) % NST, abuf[(u + 2) % NBUF], wbuf[(u + 2) % NBUF]);
                    lds_write((u + 3) % NST, abuf[(u + 3) % NBUF], wbuf[(u + 3) % NBUF]);
                }
                lds_read(u % NST, a, w);
            } else {
                barrier();
                lds_write((u + 1) & 1, abuf[(u + 1) % NBUF], wbuf[(u + 1) % NBUF]);
                lds_read(u & 1, a, w);
            }
            // bf16 with a per-tensor scale and a ragged last step: x columns
            // past Kin (the next token's first ones) are zeroed, so that an
            // infinity there adds nothing to this token
            if (XT == TQ_BF16 && LAYOUT == TQ_SCALE_TENSOR && Kin % KS != 0 && cp.j == seg_steps - 1) {
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                    for (int d = 0; d < (int)(sizeof(Frag) / 4); ++d) {
                        const int col = cp.j * KS + q * QCOLS + 2 * d;
                        a[fm][d] &= col + 1 < Kin ? 0xFFFFFFFFu : (col < Kin ? 0x0000FFFFu : 0u);
                    }
            }
            compute(cp, a, w, swbuf[u], wst0);
        } else if constexpr (kWave) {
            uint32_t w[FN];
            wave_write((u + 1) & 1, wbuf[(u + 1) % NBUF], swbuf[(u + 1) % NBUF]);
            wave_read(u & 1, w);
            compute(cp, abuf[u], w, swbuf[u], (u & 1) ? wst1 : wst0);
        } else {
            compute(cp, abuf[u], wbuf[u], swbuf[u], wst0);
        }
        cp.advance(seg_steps, KC);
    };

    Cursor ld{0, 0, 0}, cp{0, 0, 0};
#pragma unroll
    for (int u = 0; u + 1 < NBUF; ++u) {
        load(ld, abuf[u], wbuf[u], swbuf[u]);
        ld.advance(seg_steps, KC);
    }
    if constexpr (kLds) lds_write(0, abuf[0], wbuf[0]);
    if constexpr (kPair) lds_write(1, abuf[1], wbuf[1]);
    if constexpr (kWave) wave_write(0, wbuf[0], swbuf[0]);
    static_assert(!(kLds || kWave) || NBUF % 2 == 0, "stage parity follows the buffer index");
    static_assert(!kPair || (NBUF == NST && NBUF >= 6), "the ring's stage of a step is its buffer index");
    int t = 0;
    for (; t + NBUF <= total; t += NBUF) {
#pragma unroll
        for (int u = 0; u < NBUF; ++u) step(u, ld, cp, true);
    }
#pragma unroll
    for (int u = 0; u + 1 < NBUF; ++u) {   // the last total % NBUF steps, already loaded
        if (t + u < total) step(u, ld, cp, false);
    }

    // epilogue: lane holds weight row n = n0 + 16 fn + r of tokens m0 + 16 fm + 4 q + e
    float s_w = 0.0f;
    if (kDirect) s_w = ld_uniform((const float*)P.scales);
    const int64_t ybytes = (int64_t)M * N * 4;
    if (ybytes <= kYLean) {
        // y (and acc) through buffer stores: an output past M or N gets an
        // offset at or above 1 GiB, past the resource's size, so the store is
        // dropped -- one offset per row and per column, no branch per store
        // (y of at most 1 GiB)
        const __amdgpu_buffer_rsrc_t ry = rsrc(P.y, ybytes);
        const __amdgpu_buffer_rsrc_t ra = rsrc(P.acc, P.acc ? ybytes : 0);
        uint32_t colv[FN];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int n = n0 + 16 * fn + r;
            colv[fn] = n < N ? (uint32_t)n * 4u : kYPast;
        }
        // every token scale's load in flight at once
        float cm[FM][4];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = m0 + 16 * fm + 4 * q + e;
                cm[fm][e] = XT == TQ_I8 ? P.x_scale[m < M ? m : M - 1] : 1.0f;   // past M: stored nowhere
            }
        auto store_all = [&](const bool with_acc) __attribute__((always_inline)) {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = m0 + 16 * fm + 4 * q + e;
                    const uint32_t rowv = m < M ? (uint32_t)m * (uint32_t)N * 4u : kYPast;
                    const float c = kDirect ? s_w * cm[fm][e] : cm[fm][e];   // fl32(s_w * x_scale[m]), one rounding
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn) {
                        float v;
                        if (kDirect) {
                            const int a = part[fm][fn][e];
                            v = (float)a * c;
                            if (with_acc)
                                __builtin_amdgcn_raw_buffer_store_b32((uint32_t)a, ra, rowv + colv[fn], 0, 0);
                        } else {
                            v = XT == TQ_I8 ? acc[kDirect ? 0 : fm][kDirect ? 0 : fn][e] * c
                                            : acc[kDirect ? 0 : fm][kDirect ? 0 : fn][e];
                        }
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), ry, rowv + colv[fn], 0, 0);
                    }
                }
        };
        store_all(kDirect && P.acc);
        return;
    }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = m0 + 16 * fm + 4 * q + e;
            if (m >= M) continue;
            float xs = 1.0f;
            if (XT == TQ_I8) xs = P.x_scale[m];
            const float cm = kDirect ? s_w * xs : xs;   // fl32(s_w * x_scale[m]), one rounding
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

// The codebook as fp32 in LDS (codec layouts only), and the pair-code table
// of the compact base-3 codes.
template <int LAYOUT>
__device__ __forceinline__ void stage_codebook(const tq_prob_dev& P, float* cb_lds, uint8_t* b3_lut)
{
    if (LAYOUT != TQ_SCALE_CODEBOOK && LAYOUT != TQ_SCALE_CODEBOOK_B3) return;
    if (threadIdx.x < TQ_CB_SLOTS) cb_lds[threadIdx.x] = f16_to_f32(P.cb[threadIdx.x]);
    if (LAYOUT == TQ_SCALE_CODEBOOK_B3) B3Table<8>::fill(b3_lut);
    __syncthreads();
}

template <int LAYOUT>
constexpr int b3_lut_bytes() { return LAYOUT == TQ_SCALE_CODEBOOK_B3 ? B3Table<8>::kBytes : 16; }

// The prefill kernels' tables: the codebook, and the table of the compact
// codes or of the combined digits.
template <int XT, int LAYOUT, int K, int KS>
constexpr int gemm_lut_bytes() { return gemm_comb<XT, LAYOUT, K, KS>() ? D3Table::kBytes : b3_lut_bytes<LAYOUT>(); }
template <int XT, int LAYOUT, int K, int KS>
__device__ __forceinline__ void gemm_stage_tables(const tq_prob_dev& P, float* cb_lds, uint8_t* lut)
{
    if constexpr (gemm_comb<XT, LAYOUT, K, KS>()) {
        if (threadIdx.x < TQ_CB_SLOTS) cb_lds[threadIdx.x] = f16_to_f32(P.cb[threadIdx.x]);
        D3Table::fill(lut);
        __syncthreads();
    } else {
        stage_codebook<LAYOUT>(P, cb_lds, lut);
    }
}

// Waves per SIMD the register budget is sized for: the compact codec's
// few-token kernel (98 VGPRs) takes four, as its table leaves room for them.
template <int LAYOUT, int FM>
constexpr int waves_per_simd() { return LAYOUT == TQ_SCALE_CODEBOOK_B3 && FM == 1 ? 4 : TQ_GEMM_WAVES_PER_SIMD; }

template <int XT, int LAYOUT, int K, int FM, int FN, int KS, int WM>
__global__ __launch_bounds__(kThreads, (waves_per_simd<LAYOUT, FM>())) void k_gemm_single(tq_prob_dev P, int tiles_m)
{
    __shared__ float cb_lds[TQ_CB_SLOTS];
    __shared__ __attribute__((aligned(16))) uint8_t b3_lut[gemm_lut_bytes<XT, LAYOUT, K, KS>()];
    gemm_stage_tables<XT, LAYOUT, K, KS>(P, cb_lds, b3_lut);
    const int tile = blockIdx.x;
    gemm_tile<XT, LAYOUT, K, FM, FN, KS, WM>(P, tile % tiles_m, tile / tiles_m, (const LDS_AS float*)cb_lds,
                                             (const LDS_AS uint8_t*)b3_lut);
}

// Grouped: item i = (problem, tile); tiles of a problem run token-tile fastest.
template <int XT, int LAYOUT, int K, int FM, int FN, int KS, int WM>
__global__ __launch_bounds__(kThreads, (waves_per_simd<LAYOUT, FM>())) void k_gemm_grouped(const tq_prob_dev* probs, const int2* items)
{
    const int2 it = items[blockIdx.x];
    const tq_prob_dev P = ld_uniform_struct(probs + it.x);
    __shared__ float cb_lds[TQ_CB_SLOTS];
    __shared__ __attribute__((aligned(16))) uint8_t b3_lut[gemm_lut_bytes<XT, LAYOUT, K, KS>()];
    gemm_stage_tables<XT, LAYOUT, K, KS>(P, cb_lds, b3_lut);
    const int tiles_m = (P.M + 16 * FM * WM - 1) / (16 * FM * WM);
    gemm_tile<XT, LAYOUT, K, FM, FN, KS, WM>(P, it.y % tiles_m, it.y / tiles_m, (const LDS_AS float*)cb_lds,
                                             (const LDS_AS uint8_t*)b3_lut);
}

}  // namespace tqm
