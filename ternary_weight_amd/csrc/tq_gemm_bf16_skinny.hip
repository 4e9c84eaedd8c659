// libtq: bf16-activation matrix-core kernels for a few tokens (M <= 16): one
// 16-token tile per wave, 4 waves along the weight rows, 64 rows per wave.
#include "tq_gemm_impl.h"
#include "tq_gemm_kernels.h"

const tq_gemm_kernel (*tq_gemm_table_bf16_skinny())[4]
{
    static const tq_gemm_kernel t[TQ_GEMM_ROWS][4] = {
        TQ_GEMM_ROW(TQ_BF16, TQ_SCALE_TENSOR, 1, 4, 1, 4, 32, 1),
        TQ_GEMM_ROW(TQ_BF16, TQ_SCALE_GROUP_F16, 1, 4, 1, 4, 32, 1),
        TQ_GEMM_ROW(TQ_BF16, TQ_SCALE_GROUP_F16, 1, 4, 1, 4, 16, 1),
        TQ_GEMM_ROW(TQ_BF16, TQ_SCALE_CODEBOOK, 1, 4, 1, 4, 16, 1),
        TQ_GEMM_ROW_B3(1, 4, 1),
    };
    return t;
}
