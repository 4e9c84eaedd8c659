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
       TQ_GEMM_ROWS = 4 };

// Kernels of one activation type, indexed [row][K - 1]; null where unsupported.
const tq_gemm_kernel (*tq_gemm_table_i8())[4];
const tq_gemm_kernel (*tq_gemm_table_bf16())[4];
// bf16 kernels for a few tokens (M <= 16): one 16-token tile, 4 waves along the rows.
const tq_gemm_kernel (*tq_gemm_table_bf16_skinny())[4];

#define TQ_GEMM_ENTRY(XT, LAYOUT, K, FM, FN, KS, WM)                                               \
    {tqm::k_gemm_single<XT, LAYOUT, K, FM, FN, KS, WM>, tqm::k_gemm_grouped<XT, LAYOUT, K, FM, FN, KS, WM>, \
     FM, FN, KS, WM}
#define TQ_GEMM_ROW(XT, LAYOUT, FM1, FN1, FM, FN, KS, WM)                                           \
    {TQ_GEMM_ENTRY(XT, LAYOUT, 1, FM1, FN1, KS, WM), TQ_GEMM_ENTRY(XT, LAYOUT, 2, FM, FN, KS, WM),   \
     TQ_GEMM_ENTRY(XT, LAYOUT, 3, FM, FN, KS, WM), TQ_GEMM_ENTRY(XT, LAYOUT, 4, FM, FN, KS, WM)}
#define TQ_GEMM_NONE {{nullptr, nullptr, 0, 0, 0, 0}, {nullptr, nullptr, 0, 0, 0, 0}, \
                      {nullptr, nullptr, 0, 0, 0, 0}, {nullptr, nullptr, 0, 0, 0, 0}}
