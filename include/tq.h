/*
 * tq.h -- C ABI of libtq.so: packed ternary-weight matrix-vector (decode) and
 * skinny matrix-matrix (prefill) products on AMD Instinct MI355X (gfx950).
 *
 * The operation (every entry point below computes it or prepares for it):
 *
 *   y[m][n] = sum_{k<K} sum_{g<G} S_k[n][g] * sum_{i in group g} t_k[n][i] * x[m][i]
 *
 *   t_k[n][i] in {-1, 0, +1}   trit plane k of the N x Kin weight (Tritium page,
 *                              introduction: a base plane plus residual planes,
 *                              each with values -1, 0 or +1; plane 0 is the base)
 *   S_k[n][g]                  TQ_SCALE_TENSOR:   s_k, one fp32 per plane
 *                              TQ_SCALE_GROUP_F16: one f16 per plane, row and group
 *                                of g consecutive inputs (sasori page, "K and g" and
 *                                "How it works": the weight is the sum of its K
 *                                planes, each scaled group by group)
 *                              TQ_SCALE_CODEBOOK: 3^(K-1-k) * cb[idx[n][g]] -- the
 *                                balanced-ternary codec, K digits per weight, value
 *                                9 t2 + 3 t1 + t0 for K = 3, 27 levels, a codebook of
 *                                log-spaced f16 scales and one index per group
 *                                (Llama-3.1-8B-trit-uniform-d3 card, "Quantization
 *                                details")
 *   x                          activations, fp32, bf16 or int8 with a per-token scale
 *
 * The weight is stored as trits packed four to a byte, two bits each
 * (QORA-LLM-2B page, "Ternary GEMV (No Multiplication)"), codes 00 = 0,
 * 01 = +1, 10 = -1 (11 is never written and reads as 0).  The inner loops
 * only add or subtract activations; scales are applied once per group, or
 * once at the end for a per-tensor scale (same section).
 *
 * Conventions for every call:
 *  - A weight is N x Kin (out_features x in_features), as a Linear layer's
 *    weight; x is [M][Kin] row-major and y is [M][N] row-major fp32.
 *  - Pointers marked "device" are HIP device pointers owned by the caller;
 *    the library keeps no reference after the call's work has run and
 *    allocates no device memory (tq_ternarize_noalloc's fixed scratch array
 *    aside, see there).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue
 *    their kernels on it and return without waiting, except tq_pack (see
 *    there) and tq_gemv_grouped_prepare.
 *  - Alignment (TQ_ERR_ALIGN otherwise): blobs, tq_pack's trits and
 *    tq_act_quant_int8's x and xq 16 bytes; every other device array 4 bytes
 *    (2 for f16 codebooks).  Outputs must not alias inputs.
 *  - Argument, shape, alignment and support errors are returned before
 *    anything is enqueued.  A failed launch returns TQ_ERR_DEVICE.  Details
 *    of the last error of the calling thread are in tq_last_error().
 *  - The calls are thread-safe; calls that overlap on one stream are ordered
 *    by the stream.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_ABI_VERSION 1

typedef enum tq_status {
    TQ_OK = 0,
    TQ_ERR_ARG = 1,          /* null pointer, bad enum, negative size            */
    TQ_ERR_SHAPE = 2,        /* Kin % 16, Kin % g, size limits                   */
    TQ_ERR_ALIGN = 3,        /* device pointer not 16-byte aligned               */
    TQ_ERR_VALUE = 4,        /* tq_pack: trit outside {-1,0,1}, index >= n_cb,
                                non-finite scale                                  */
    TQ_ERR_UNSUPPORTED = 5,  /* valid but not provided (see each call)           */
    TQ_ERR_DEVICE = 6        /* HIP runtime or launch failure                     */
} tq_status;

typedef enum tq_scale_layout {
    TQ_SCALE_TENSOR = 0,     /* canonical scales: fp32 s[K]                           */
    TQ_SCALE_GROUP_F16 = 1,  /* canonical scales: f16 bits s[K][N][Kin/g]             */
    TQ_SCALE_CODEBOOK = 2,   /* canonical scales: uint8 idx[N][Kin/g] into f16 cb[]   */
    TQ_SCALE_CODEBOOK_B3 = 3 /* the codec of TQ_SCALE_CODEBOOK (same canonical arrays,
                                same results) with its codes packed compactly in base 3:
                                the K = 3 digits of a weight are one base-27 value v in
                                [-13, 13], and two neighbouring weights one 10-bit code
                                (v0 mod 27) + 27 (v1 mod 27) < 729, so 5 bits per weight
                                where the two-bit planes take 6 (the Tritium page's
                                feature list names "compact B3 packing"; this is our
                                reading of it for the codec).  planes must be 3.
                                Decode and prefill take bf16 activations only.         */
} tq_scale_layout;

typedef enum tq_dtype {
    TQ_F32 = 0,
    TQ_BF16 = 1,             /* bits of bfloat16 values, uint16 storage                */
    TQ_I8 = 2,               /* int8 values with an fp32 scale per token (row of x)  */
    TQ_F32_Q8 = 3            /* fp32 values quantised per token to int8 inside the
                                product, by the rule of tq_act_quant_int8, then
                                accumulated as TQ_I8 (bit-identical to the two calls);
                                tq_gemv / tq_gemv_grouped only, M * Kin <= 65536      */
} tq_dtype;

/* Shape and format of one packed weight. */
typedef struct tq_weight_desc {
    int32_t planes;          /* K, 1..4: trit planes, or digits of the codec          */
    int32_t group;           /* g in {16,32,64,128,256} for GROUP_F16 and CODEBOOK;
                                ignored for TENSOR                                      */
    int32_t scale_layout;    /* tq_scale_layout                                       */
    int32_t n_codebook;      /* CODEBOOK: entries 1..32 (27 for the d = 3 codec);
                                ignored otherwise                                       */
    int64_t out_features;    /* N, 0..2^24                                            */
    int64_t in_features;     /* Kin, 0..65536, a multiple of 16 and of g              */
} tq_weight_desc;

int32_t     tq_abi_version(void);
const char* tq_status_string(int32_t status);
/* Text of the last error returned on the calling thread ("" if none). */
const char* tq_last_error(void);

/*
 * Bytes of the packed blob for `desc` (header, trit planes, scales or codebook
 * and indices).  The trit planes take K * N * Kin / 4 bytes for N and Kin
 * multiples of 64 (padding rounds each up to 64 otherwise); GROUP_F16 scales
 * take 2 bytes per plane, row and group, so the physical bits per weight
 * approach 2K + 16K/g (the bpw column of the sasori page's "K and g" table).
 * Pure host arithmetic; needs no GPU.
 */
tq_status tq_packed_size(const tq_weight_desc* desc, size_t* bytes);

/*
 * Pack canonical planes and scales into the opaque device blob.
 *   trits     device int8 [K][N][Kin], values -1, 0, +1 (digits for CODEBOOK,
 *             plane 0 the most significant)
 *   scales    device, canonical layout of desc->scale_layout (see the enum)
 *   codebook  device f16 bits [n_codebook] for CODEBOOK, NULL otherwise
 *   blob      device, tq_packed_size(desc) bytes, written in full
 * Validates every value on the device and synchronizes `stream` to report
 * TQ_ERR_VALUE (the blob's contents are then unspecified).  Offline step: not
 * meant for a hot loop.
 */
tq_status tq_pack(const tq_weight_desc* desc, const int8_t* trits, const void* scales,
                  const uint16_t* codebook, void* blob, void* stream);

/*
 * Inverse of tq_pack: the canonical arrays back from a blob (device pointers,
 * same layouts as tq_pack's inputs; codebook may be NULL).  Asynchronous.
 */
tq_status tq_unpack(const tq_weight_desc* desc, const void* blob, int8_t* trits, void* scales,
                    uint16_t* codebook, void* stream);

/*
 * Per-token absmax int8 quantisation of x [M][Kin] (x_type TQ_F32 or TQ_BF16):
 *   a_m = max_i |x[m][i]|;   a_m = 0 -> xq = 0 and x_scale[m] = 0;
 *   otherwise inv = fl32(127 / a_m), xq[m][i] = clamp(rne(fl32(x * inv)), -127, 127)
 *   and x_scale[m] = fl32(a_m / 127).
 * xq device int8 [M][Kin], x_scale device fp32 [M].  Non-finite x: unspecified.
 */
tq_status tq_act_quant_int8(int64_t M, int64_t in_features, int32_t x_type, const void* x,
                            int8_t* xq, float* x_scale, void* stream);

/* One activation matrix for tq_act_quant_int8_batch. */
typedef struct tq_act_segment {
    int64_t M;                    /* tokens (rows)                              */
    int64_t in_features;          /* Kin, a multiple of 16                      */
    int32_t x_type;               /* TQ_F32 or TQ_BF16                          */
    int32_t reserved;
    const void* x;                /* device [M][Kin], 16-byte aligned           */
    int8_t* xq;                   /* device [M][Kin], 16-byte aligned           */
    float* x_scale;               /* device [M]                                 */
} tq_act_segment;

#define TQ_ACT_MAX_SEGMENTS 16

/*
 * tq_act_quant_int8 for up to TQ_ACT_MAX_SEGMENTS matrices in one launch
 * (e.g. the inputs of every projection of a layer stack, grouped by width).
 * `segments` is a host array; same per-token rule and results.
 */
tq_status tq_act_quant_int8_batch(const tq_act_segment* segments, int32_t count, void* stream);

/*
 * Decode product for M <= 16 tokens (vector-ALU kernels: unpack, add/subtract,
 * scale per group; up to 4 tokens per pass over the codes, one launch per
 * slice of 4 tokens beyond that).  With TQ_BF16 and M >= 3 (5 for the two
 * codebook layouts), or TQ_I8, M >= 2 and groups of 64 or more columns (or
 * a per-tensor scale), and x 16-byte aligned, the product runs on the
 * matrix cores instead, as tq_gemm does, one pass over the codes for all M
 * tokens; the results meet the same bound (TQ_I8 with one plane and a
 * per-tensor scale: the same bits).
 *   x         device [M][Kin] of x_type
 *   x_scale   device fp32 [M], TQ_I8 only (from tq_act_quant_int8), else unused
 *             (TQ_F32_Q8 computes the per-token scales itself)
 *   y         device fp32 [M][N]
 *   acc       optional device int32 [M][N]: the integer accumulator, only for
 *             TQ_I8 / TQ_F32_Q8 with TQ_SCALE_TENSOR and K = 1
 *             (TQ_ERR_UNSUPPORTED otherwise)
 * TQ_I8 and TQ_F32_Q8 with TQ_SCALE_TENSOR and K = 1 are bit exact:
 *   y = fl32(float(acc) * fl32(s_w * x_scale[m])).
 * Other combinations accumulate in fp32.  M = 0 or N = 0 is a no-op.
 */
tq_status tq_gemv(const tq_weight_desc* desc, const void* blob, int64_t M, int32_t x_type,
                  const void* x, const float* x_scale, float* y, int32_t* acc, void* stream);

/*
 * Prefill product for any M (matrix-core kernels: the trits of each 16 x 16
 * weight tile are decoded in registers to the MFMA operand type, the MFMA
 * accumulates one plane and group at a time, and the group's scale is applied
 * once when the group ends).  Same arguments and results as tq_gemv, with:
 *   x_type    TQ_I8 (int8 MFMA, int32 accumulate) or TQ_BF16 (bf16 MFMA,
 *             fp32 accumulate); TQ_F32 and TQ_F32_Q8 are TQ_ERR_UNSUPPORTED
 *   layout    TQ_I8: TQ_SCALE_TENSOR, or TQ_SCALE_GROUP_F16 with g a multiple of
 *             the 64-column int8 MFMA step.  TQ_BF16: every layout and group
 *             size (32-column steps where g allows, else 16-column steps, one
 *             per group of 16).  Other combinations are TQ_ERR_UNSUPPORTED.
 *   x         device, 16-byte aligned (rows are read 16 bytes at a time)
 *   M         0 .. 2^24
 * TQ_I8 with TQ_SCALE_TENSOR and K = 1 is bit exact, as in tq_gemv:
 *   acc = sum_i t[n][i] * xq[m][i] (int32), y = fl32(float(acc) * fl32(s_w * x_scale[m])).
 */
tq_status tq_gemm(const tq_weight_desc* desc, const void* blob, int64_t M, int32_t x_type,
                  const void* x, const float* x_scale, float* y, int32_t* acc, void* stream);

/*
 * Many decode products in one launch (a whole layer stack).  All problems
 * must share K, scale layout, g (when used), x_type and M.
 */
typedef struct tq_problem {
    const tq_weight_desc* desc;   /* host pointer                              */
    const void* blob;             /* device                                    */
    const void* x;                /* device [M][Kin]                           */
    const float* x_scale;         /* device [M] for TQ_I8, else NULL           */
    float* y;                     /* device [M][N]                             */
    int32_t* acc;                 /* optional, as in tq_gemv                   */
} tq_problem;

/* Filled by tq_gemv_grouped_prepare; plain data, may be copied. */
typedef struct tq_grouped_plan {
    const void* workspace;        /* device table written by prepare           */
    int64_t n_items;              /* 64-row blocks over all problems           */
    int32_t family;               /* kernel family selected at prepare         */
    int32_t x_type;
    int32_t M;
    int32_t waves;                /* in: 0 or 1, 2, 4, 8, 16; out: waves that
                                     split the columns of one 64-row block      */
    int32_t row_blocks;           /* in: 0 or 1, 2, 4, 8, 16; out: 64-row blocks
                                     per workgroup (waves * row_blocks <= 16)   */
    int32_t n_problems;
    int32_t x_lds_bytes;          /* LDS for in-kernel quantised activations   */
    int32_t mode;                 /* 0: an item per workgroup; 1: an item per
                                     wave, the token slices of one row block in
                                     one workgroup (set by prepare, bf16)      */
} tq_grouped_plan;

/* Device workspace bytes that tq_gemv_grouped_prepare needs for these problems. */
tq_status tq_gemv_grouped_workspace_size(const tq_problem* problems, int32_t count, int64_t M,
                                         size_t* bytes);

/*
 * Validate the problems, write their descriptor table and the work list into
 * `workspace` (device, caller-owned) and fill `plan`.  With TQ_BF16, M >= 3
 * (5 for the codebook layouts), or TQ_I8, M >= 2 and every problem's groups
 * of 64 columns or more (or a per-tensor scale), every x 16-byte aligned and
 * no shape hint in `plan`, the plan is a matrix-core plan (as from
 * tq_gemm_grouped_prepare).  Otherwise the run is one launch
 * with one workgroup per item, an item being `row_blocks` consecutive 64-row
 * blocks of one problem, each split over `waves` waves; items are ordered
 * longest first.  On entry plan->waves and plan->row_blocks choose the shape
 * (0 = default: 4 waves, 1 block; with TQ_F32_Q8 1 wave, 4 blocks, so that a
 * workgroup quantises its activations once for four blocks; with TQ_I8 and
 * M > 1 2 waves, 2 blocks for one plane and a per-tensor scale, else 1 wave,
 * 4 blocks; with TQ_BF16 1 wave, 16 blocks, or 2 waves, 4 blocks for M > 1,
 * so that the blocks share the workgroup's trit table).  The
 * decode kernels take up to 4 tokens per pass over the codes: with more, each
 * problem is cut into slices of 4 tokens.
 * With TQ_BF16 (per-tensor or f16 group scales) and no shape hint an item is
 * then one 64-row block of one slice per wave, the slices of a row block in
 * one workgroup of 16 waves; otherwise the slices' workgroups are placed to
 * run on one XCD together.  Copies host->device on `stream` and synchronizes
 * it.
 */
tq_status tq_gemv_grouped_prepare(const tq_problem* problems, int32_t count, int64_t M,
                                  int32_t x_type, void* workspace, size_t workspace_bytes,
                                  tq_grouped_plan* plan, void* stream);

/*
 * As tq_gemv_grouped_prepare, but problem i has its own token count
 * tokens[i] (host array of `count`, each 0..16): x is tokens[i] x Kin and y
 * tokens[i] x N.  This is the expert-grouped decode of a mixture-of-experts
 * layer: every expert's matrix is fit on its own (sasori page, "How it works
 * & paper"), so each expert is one problem with its own blob, and the tokens
 * the router sent to it are gathered into its x.  A problem with no tokens
 * takes no workgroup (its pointers may then be NULL).  With TQ_BF16 and a
 * mean count of at least 3 (5 for the codebook layouts) over the problems
 * that have tokens, or TQ_I8 and a mean count of at least 2 (groups of 64
 * columns or more), every x 16-byte
 * aligned and no shape hint in `plan`, the plan is a matrix-core plan whose
 * tiles cover each problem's own count; otherwise the vector-ALU kernels take
 * up to 4 tokens per pass and a problem with more is cut into slices of 4 (as
 * in tq_gemv_grouped_prepare).  The workspace is
 * tq_gemv_grouped_workspace_size's with M = the largest count.  More than 16 tokens for one expert: split them over
 * several problems that share the blob.  Errors as tq_gemv_grouped_prepare,
 * plus TQ_ERR_ARG for a NULL `tokens` with count > 0 or a negative count and
 * TQ_ERR_UNSUPPORTED for a count above 16.
 */
tq_status tq_gemv_grouped_prepare_tokens(const tq_problem* problems, const int32_t* tokens,
                                         int32_t count, int32_t x_type, void* workspace,
                                         size_t workspace_bytes, tq_grouped_plan* plan, void* stream);

/* One launch computing every problem of the plan.  Asynchronous. */
tq_status tq_gemv_grouped_run(const tq_grouped_plan* plan, void* stream);

/*
 * Many prefill products (tq_gemm) in one launch, e.g. every projection of a
 * layer stack.  All problems must share K, scale layout and x_type; M is
 * common.  The work list holds one item per output tile (16 tokens x 256 rows
 * for TQ_BF16 with M <= 16, else 128 x 128), longest problems first.  The
 * plan is the decode one's struct: on return waves = 4 and row_blocks =
 * 64-row blocks per tile; tq_gemv_grouped_run runs it as well.
 */
tq_status tq_gemm_grouped_workspace_size(const tq_problem* problems, int32_t count, int64_t M,
                                         int32_t x_type, size_t* bytes);
/* Validate, write the problem table and work list to `workspace` (device),
   fill `plan`.  Copies host->device on `stream` and synchronizes it. */
tq_status tq_gemm_grouped_prepare(const tq_problem* problems, int32_t count, int64_t M,
                                  int32_t x_type, void* workspace, size_t workspace_bytes,
                                  tq_grouped_plan* plan, void* stream);
/* One launch computing every problem of the plan.  Asynchronous. */
tq_status tq_gemm_grouped_run(const tq_grouped_plan* plan, void* stream);

/*
 * Ternarizer: fit a dense fp32 weight w [N][Kin] (device) into the canonical
 * arrays that tq_pack takes -- trits int8 [K][N][Kin] and scales (device) --
 * before packing.  Each matrix is fit on its own, weight-only (sasori page,
 * "How it works & paper": a sum of K per-group-scaled trit-planes; d3 card,
 * "Quantization details": uniform quantisation onto 27 levels with a
 * 27-entry log-spaced scale codebook).  By scale layout:
 *
 *  TQ_SCALE_GROUP_F16, TQ_SCALE_TENSOR -- greedy residual planes.  R = w; for
 *  k = 0 .. K-1, per group (g inputs of a row; the whole tensor for TENSOR):
 *    a = mean |R|;  t = sign(R) where |R| > a / 2, else 0;
 *    s = mean of |R| where t != 0 (the least-squares scale of t; 0 if none);
 *    R = fl(R - s t).
 *  Sums are fp64 in index order (TENSOR: each row, then the row sums in row
 *  order), divided in fp64 and rounded to fp32; GROUP_F16 rounds s to f16
 *  (ties to even, saturating at 65504) and uses the rounded value after.
 *  No plane increases any group's squared error.
 *
 *  TQ_SCALE_CODEBOOK -- codebook (device f16 [n_codebook], positive and
 *  ascending, checked) per group of g: a = max |w|, L = (3^K - 1) / 2
 *  levels a side, idx = the first entry >= fl(a / L) (the last if none),
 *  q = clamp(rint(fl(w / cb[idx])), -L, L) written as balanced-ternary
 *  digits, plane p holding the digit of 3^(K-1-p) (p = 0: t2 for K = 3);
 *  scales = idx as uint8 [N][Kin / g].
 *
 * The results equal the CPU oracle's bit for bit.  workspace: device bytes
 * from tq_ternarize_workspace_size (TENSOR only; NULL and 0 otherwise).
 * Non-finite weights are out of contract.  An offline call: CODEBOOK reads
 * the codebook back and synchronizes `stream`; the rest is asynchronous.
 */
tq_status tq_ternarize_workspace_size(const tq_weight_desc* desc, size_t* bytes);
tq_status tq_ternarize(const tq_weight_desc* desc, const float* w, const uint16_t* codebook, int8_t* trits,
                       void* scales, void* workspace, size_t workspace_bytes, void* stream);

/*
 * tq_ternarize for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops, harnesses that forbid hipMalloc): the
 * same fit and the same results, bit for bit, with no workspace argument.
 * TQ_SCALE_TENSOR keeps its per-row partial sums in a scratch array that
 * the library holds in device memory, one copy per GPU for the life of the
 * process (4 MiB): at most 262144 rows (TQ_ERR_UNSUPPORTED beyond, before
 * anything is enqueued).  Every row the fit reads is written first in the
 * same call, so nothing in the scratch has to start at zero; it keeps the
 * last call's contents.  All calls on one GPU share that array: calls that
 * may overlap on one GPU (other streams, other threads) race and must be
 * ordered by the caller.  The other layouts use no scratch.  No call here
 * allocates; the rest is as tq_ternarize.
 */
tq_status tq_ternarize_noalloc(const tq_weight_desc* desc, const float* w, const uint16_t* codebook,
                               int8_t* trits, void* scales, void* stream);

/*
 * Decode chain: BitNet b1.58 layers run back to back for one token in one
 * persistent launch, in the order of the QORA-LLM-2B page's "SubLN Pattern"
 * listing (head counts from its "Architecture" table).  Per layer, with x
 * the token's hidden state:
 *
 *   h  = RMSNorm(x, norm[0]);            q, k, v = W_q h, W_k h, W_v h
 *   a  = attention(q, k, v);             x1 = x + W_o RMSNorm(a, norm[1])
 *   h2 = RMSNorm(x1, norm[2]);           g, u = W_gate h2, W_up h2
 *   x  = x1 + W_down RMSNorm(relu2(g) * u, norm[3]),   relu2(z) = max(0, z)^2
 *
 * The token is at position 0: attention over its single cached key has
 * softmax weight 1, so each query head's output is the value vector of its
 * KV group (query head h reads KV head h / (n_heads / n_kv_heads)); q and k
 * do not reach x but are computed and returned, as a decode step stores its
 * keys and values.
 *
 * Arithmetic, step by step (the CPU oracle's, bit for bit):
 *  - every ternary linear runs on the int8 path: its input is quantised per
 *    token by tq_act_quant_int8's rule, and its output is
 *    fl(float(acc) * fl(s_w * s_x)) with acc the exact int32 sum;
 *  - RMSNorm: the sum of squares in fp64, the mean rounded once to fp32,
 *    r = fl(1 / fl(sqrt(fl(mean + eps)))), out_i = fl(fl(v_i * r) * w_i);
 *  - relu2(g) * u = fl(fl(g' * g') * u), g' = max(g, 0); the residual adds
 *    are single fp32 adds.
 * The fp64 sums of squares are added in another order than the oracle's;
 * the fp32 mean can differ only when the exact sum lies within ~1e-14
 * relative of an fp32 rounding boundary.
 */
typedef struct tq_bitnet_dims {
    int32_t hidden;               /* model width; n_heads * head_dim == hidden  */
    int32_t intermediate;         /* FFN width                                  */
    int32_t n_heads;              /* query heads                                */
    int32_t n_kv_heads;           /* KV heads, dividing n_heads                 */
    int32_t head_dim;
    float eps;                    /* RMSNorm epsilon                            */
} tq_bitnet_dims;

/* One layer's weights, all device pointers owned by the caller. */
typedef struct tq_bitnet_layer {
    /* blobs packed by tq_pack with planes = 1, TQ_SCALE_TENSOR, shapes (N x Kin)
       q: n_heads*head_dim x hidden, k and v: n_kv_heads*head_dim x hidden,
       o: hidden x n_heads*head_dim, gate and up: intermediate x hidden,
       down: hidden x intermediate -- in that order                            */
    const void* w[7];
    /* fp32 RMSNorm weights: input [hidden], attention-sub [hidden],
       post-attention [hidden], FFN-sub [intermediate]                         */
    const float* norm[4];
} tq_bitnet_layer;

/* Filled by tq_bitnet_chain_prepare; plain data, may be copied. */
typedef struct tq_chain_plan {
    void* workspace;              /* device: layer table and chain state        */
    int32_t n_layers;
    int32_t workgroups;           /* in: 0 (default) or a count; out: the grid  */
    tq_bitnet_dims dims;
    int32_t reserved[4];
} tq_chain_plan;

/* Device workspace bytes that tq_bitnet_chain_prepare needs. */
tq_status tq_bitnet_chain_workspace_size(const tq_bitnet_dims* dims, int32_t n_layers, size_t* bytes);

/*
 * Validate the dimensions and the layers (`layers` is a host array of
 * n_layers; each blob's header is read back to check its shape and format),
 * write the layer table into `workspace` (device, caller-owned, kept for the
 * plan's lifetime) and clear the chain state.  Widths up to 8192, each a
 * multiple of 16; head_dim a multiple of 4.  plan->workgroups on entry: 0 for one workgroup per two
 * compute units, else the grid to use (at most what fits the GPU at once).
 * Copies host->device on `stream` and synchronizes it.
 */
tq_status tq_bitnet_chain_prepare(const tq_bitnet_dims* dims, const tq_bitnet_layer* layers,
                                  int32_t n_layers, void* workspace, size_t workspace_bytes,
                                  tq_chain_plan* plan, void* stream);

/*
 * Run every layer of the plan on one token.  x: device fp32 [hidden], the
 * hidden state entering the first layer on entry and leaving the last on
 * return.  qkv: optional device fp32 [n_layers][(n_heads + 2 n_kv_heads) *
 * head_dim], each layer's q, k and v.  One cooperative launch (all
 * workgroups resident; a phase waits until the output blocks it reads have
 * been written) after a small reset launch.  Asynchronous; runs on one
 * stream at a time per workspace.
 */
tq_status tq_bitnet_chain_run(const tq_chain_plan* plan, float* x, float* qkv, void* stream);

/*
 * Synchronize `stream` and report whether the plan's last run completed:
 * TQ_ERR_DEVICE if a wait between phases gave up (the grid was not all
 * resident) -- x is then undefined.
 */
tq_status tq_bitnet_chain_status(const tq_chain_plan* plan, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
