// libtq: bf16-activation prefill kernels (bf16 MFMA, fp32 accumulate).
#include "tq_gemm_impl.h"
#include "tq_gemm_kernels.h"

// 32-column steps (v_mfma_f32_16x16x32_bf16) where the group allows, else
// 16-column steps (v_mfma_f32_16x16x16_bf16): groups of 16 and the codec.
const tq_gemm_kernel (*tq_gemm_table_bf16())[4]
{
    static const tq_gemm_kernel t[TQ_GEMM_ROWS][4] = {
        TQ_GEMM_ROW(TQ_BF16, TQ_SCALE_TENSOR, 4, 4, 4, 4, 32, 2),
        TQ_GEMM_ROW(TQ_BF16, TQ_SCALE_GROUP_F16, 4, 4, 4, 4, 32, 2),
        TQ_GEMM_ROW(TQ_BF16, TQ_SCALE_GROUP_F16, 4, 4, 4, 4, 16, 2),
        TQ_GEMM_ROW(TQ_BF16, TQ_SCALE_CODEBOOK, 4, 4, 4, 4, 16, 2),
        TQ_GEMM_ROW_B3(4, 4, 2),
    };
    return t;
}
