// libtq: int8-activation matrix-core kernels for a few tokens (M <= 16): one
// 16-token tile, 4 waves along the weight rows, 64 rows per wave, a whole
// 64-column chunk of every plane per step, one v_mfma_i32_16x16x64_i8 per
// plane and 16-row tile (tq_gemm_skinny.h).  Groups must be whole steps (64
// columns and more), as for the int8 prefill kernels.
#include "tq_gemm_kernels.h"
#include "tq_gemm_skinny.h"

const tq_gemm_kernel (*tq_gemm_table_i8_skinny())[4]
{
    static const tq_gemm_kernel t[TQ_GEMM_ROWS][4] = {
        TQ_SKINNY_ROW(TQ_I8, TQ_SCALE_TENSOR, 64),
        TQ_SKINNY_ROW(TQ_I8, TQ_SCALE_GROUP_F16, 64),
        TQ_GEMM_NONE,
        TQ_GEMM_NONE,
        TQ_GEMM_NONE,
    };
    return t;
}

const tq_gemm_kernel (*tq_gemm_table_i8_skinny_wide())[4]
{
    static const tq_gemm_kernel t[TQ_GEMM_ROWS][4] = {
        {TQ_SKINNY_WIDE_ENTRY(TQ_I8, TQ_SCALE_TENSOR, 1, 64), TQ_SKINNY_ENTRY(TQ_I8, TQ_SCALE_TENSOR, 2, 64),
         TQ_SKINNY_ENTRY(TQ_I8, TQ_SCALE_TENSOR, 3, 64), TQ_SKINNY_ENTRY(TQ_I8, TQ_SCALE_TENSOR, 4, 64)},
        TQ_SKINNY_ROW(TQ_I8, TQ_SCALE_GROUP_F16, 64),
        TQ_GEMM_NONE,
        TQ_GEMM_NONE,
        TQ_GEMM_NONE,
    };
    return t;
}
