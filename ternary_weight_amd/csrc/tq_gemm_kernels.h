#pragma once
// libtq: the prefill kernel families as the host dispatch sees them.
#include "tq_internal.h"

typedef void (*tq_gemm_single_fn)(tq_prob_dev, int);
typedef void (*tq_gemm_grouped_fn)(const tq_prob_dev*, const int2*);

struct tq_gemm_kernel {
    tq_gemm_single_fn single;
    tq_gemm_grouped_fn grouped;
    int fm, fn;                  // 16 x 16 tiles per wave (tokens, weight rows)
    int step;                    // columns per MFMA step
    int wm;                      // waves along the tokens (2 x 2 or 1 x 4 waves)
};

// Rows of a kernel table: the scale layout and, for bf16, the MFMA step.
enum { TQ_GEMM_ROW_TENSOR = 0, TQ_GEMM_ROW_GROUP = 1, TQ_GEMM_ROW_GROUP16 = 2, TQ_GEMM_ROW_CODEBOOK = 3,
       TQ_GEMM_ROW_CODEBOOK_B3 = 4, TQ_GEMM_ROWS = 5 };

// Kernels of one activation type, indexed [row][K - 1]; null where unsupported.
const tq_gemm_kernel (*tq_gemm_table_i8())[4];
const tq_gemm_kernel (*tq_gemm_table_bf16())[4];
// Kernels for a few tokens (M <= 16): one 16-token tile, 4 waves along the rows.
const tq_gemm_kernel (*tq_gemm_table_bf16_skinny())[4];
const tq_gemm_kernel (*tq_gemm_table_i8_skinny())[4];
// int8 with 8 to 16 tokens: one plane with a per-tensor scale on the wide
// kernels (two 64-row blocks per wave), the rest as with fewer tokens.
const tq_gemm_kernel (*tq_gemm_table_i8_skinny_wide())[4];

#define TQ_GEMM_ENTRY(XT, LAYOUT, K, FM, FN, KS, WM)                                               \
    {tqm::k_gemm_single<XT, LAYOUT, K, FM, FN, KS, WM>, tqm::k_gemm_grouped<XT, LAYOUT, K, FM, FN, KS, WM>, \
     FM, FN, KS, WM}
#define TQ_GEMM_ROW(XT, LAYOUT, FM1, FN1, FM, FN, KS, WM)                                           \
    {TQ_GEMM_ENTRY(XT, LAYOUT, 1, FM1, FN1, KS, WM), TQ_GEMM_ENTRY(XT, LAYOUT, 2, FM, FN, KS, WM),   \
     TQ_GEMM_ENTRY(XT, LAYOUT, 3, FM, FN, KS, WM), TQ_GEMM_ENTRY(XT, LAYOUT, 4, FM, FN, KS, WM)}
#define TQ_GEMM_NONE_ENTRY {nullptr, nullptr, 0, 0, 0, 0}
#define TQ_GEMM_NONE {TQ_GEMM_NONE_ENTRY, TQ_GEMM_NONE_ENTRY, TQ_GEMM_NONE_ENTRY, TQ_GEMM_NONE_ENTRY}
// The compact base-3 codec: planes = 3 (the table's index), one combined
// value per weight in the kernel (its K = 1), 16-column steps.
#define TQ_GEMM_ROW_B3(FM, FN, WM) \
    {TQ_GEMM_NONE_ENTRY, TQ_GEMM_NONE_ENTRY, TQ_GEMM_ENTRY(TQ_BF16, TQ_SCALE_CODEBOOK_B3, 1, FM, FN, 16, WM), \
     TQ_GEMM_NONE_ENTRY}
// The few-token kernels (tq_gemm_skinny.h): one 16-token tile, 4 waves of
// 64 rows each, a 64-column chunk of every plane per step; the wide ones
// 128 rows per wave.
#define TQ_SKINNY_ENTRY(XT, LAYOUT, K, KS) \
    {tqm::k_gemm_skinny<XT, LAYOUT, K, KS>, tqm::k_gemm_skinny_grouped<XT, LAYOUT, K, KS>, 1, 4, KS, 1}
#define TQ_SKINNY_WIDE_ENTRY(XT, LAYOUT, K, KS) \
    {tqm::k_gemm_skinny_wide<XT, LAYOUT, K, KS>, tqm::k_gemm_skinny_wide_grouped<XT, LAYOUT, K, KS>, 1, 8, KS, 1}
#define TQ_SKINNY_ROW(XT, LAYOUT, KS)                                                                     \
    {TQ_SKINNY_ENTRY(XT, LAYOUT, 1, KS), TQ_SKINNY_ENTRY(XT, LAYOUT, 2, KS), TQ_SKINNY_ENTRY(XT, LAYOUT, 3, KS), \
     TQ_SKINNY_ENTRY(XT, LAYOUT, 4, KS)}
#define TQ_SKINNY_ROW_B3 \
    {TQ_GEMM_NONE_ENTRY, TQ_GEMM_NONE_ENTRY, TQ_SKINNY_ENTRY(TQ_BF16, TQ_SCALE_CODEBOOK_B3, 1, 16), TQ_GEMM_NONE_ENTRY}
