#pragma once
// libtq: the prefill kernel families as the host dispatch sees them.
#include "tq_internal.h"

typedef void (*tq_gemm_single_fn)(tq_prob_dev, int);
typedef void (*tq_gemm_grouped_fn)(const tq_prob_dev*, const int2*);

struct tq_gemm_kernel {
    tq_gemm_single_fn single;
    tq_gemm_grouped_fn grouped;
    int fm, fn;                  // 16 x 16 tiles per wave (tokens, weight rows)
};

// Kernels of one activation type, indexed [layout (TENSOR, GROUP_F16)][K - 1].
const tq_gemm_kernel (*tq_gemm_table_i8())[4];
const tq_gemm_kernel (*tq_gemm_table_bf16())[4];

#define TQ_GEMM_TABLE(NAME, XT, FM_T, FN_T, FM_G, FN_G)                                                   \
    const tq_gemm_kernel (*NAME())[4]                                                                     \
    {                                                                                                     \
        static const tq_gemm_kernel t[2][4] = {                                                           \
            {{tqm::k_gemm_single<XT, TQ_SCALE_TENSOR, 1, FM_T, FN_T>,                                     \
              tqm::k_gemm_grouped<XT, TQ_SCALE_TENSOR, 1, FM_T, FN_T>, FM_T, FN_T},                      \
             {tqm::k_gemm_single<XT, TQ_SCALE_TENSOR, 2, FM_G, FN_G>,                                     \
              tqm::k_gemm_grouped<XT, TQ_SCALE_TENSOR, 2, FM_G, FN_G>, FM_G, FN_G},                      \
             {tqm::k_gemm_single<XT, TQ_SCALE_TENSOR, 3, FM_G, FN_G>,                                     \
              tqm::k_gemm_grouped<XT, TQ_SCALE_TENSOR, 3, FM_G, FN_G>, FM_G, FN_G},                      \
             {tqm::k_gemm_single<XT, TQ_SCALE_TENSOR, 4, FM_G, FN_G>,                                     \
              tqm::k_gemm_grouped<XT, TQ_SCALE_TENSOR, 4, FM_G, FN_G>, FM_G, FN_G}},                     \
            {{tqm::k_gemm_single<XT, TQ_SCALE_GROUP_F16, 1, FM_G, FN_G>,                                  \
              tqm::k_gemm_grouped<XT, TQ_SCALE_GROUP_F16, 1, FM_G, FN_G>, FM_G, FN_G},                   \
             {tqm::k_gemm_single<XT, TQ_SCALE_GROUP_F16, 2, FM_G, FN_G>,                                  \
              tqm::k_gemm_grouped<XT, TQ_SCALE_GROUP_F16, 2, FM_G, FN_G>, FM_G, FN_G},                   \
             {tqm::k_gemm_single<XT, TQ_SCALE_GROUP_F16, 3, FM_G, FN_G>,                                  \
              tqm::k_gemm_grouped<XT, TQ_SCALE_GROUP_F16, 3, FM_G, FN_G>, FM_G, FN_G},                   \
             {tqm::k_gemm_single<XT, TQ_SCALE_GROUP_F16, 4, FM_G, FN_G>,                                  \
              tqm::k_gemm_grouped<XT, TQ_SCALE_GROUP_F16, 4, FM_G, FN_G>, FM_G, FN_G}}};                 \
        return t;                                                                                         \
    }
