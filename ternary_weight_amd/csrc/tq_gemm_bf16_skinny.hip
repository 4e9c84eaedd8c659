// libtq: bf16-activation matrix-core kernels for a few tokens (M <= 16): one
// 16-token tile, 4 waves along the weight rows, 64 rows per wave, a whole
// 64-column chunk of every plane per step (tq_gemm_skinny.h).
#include "tq_gemm_kernels.h"
#include "tq_gemm_skinny.h"

const tq_gemm_kernel (*tq_gemm_table_bf16_skinny())[4]
{
    static const tq_gemm_kernel t[TQ_GEMM_ROWS][4] = {
        TQ_SKINNY_ROW(TQ_BF16, TQ_SCALE_TENSOR, 32),
        TQ_SKINNY_ROW(TQ_BF16, TQ_SCALE_GROUP_F16, 32),
        TQ_SKINNY_ROW(TQ_BF16, TQ_SCALE_GROUP_F16, 16),
        TQ_SKINNY_ROW(TQ_BF16, TQ_SCALE_CODEBOOK, 16),
        TQ_SKINNY_ROW_B3,
    };
    return t;
}
