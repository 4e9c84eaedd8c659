// libtq: int8-activation prefill kernels (int8 MFMA, int32 accumulate).
#include "tq_gemm_impl.h"
#include "tq_gemm_kernels.h"

// 4 x 4 tiles per wave (a 128 x 128 workgroup tile) at two waves per SIMD:
// measured faster than 4 x 8 or 8 x 4 at one wave per SIMD, and than smaller
// tiles, which load more per MFMA.
const tq_gemm_kernel (*tq_gemm_table_i8())[4]
{
    static const tq_gemm_kernel t[TQ_GEMM_ROWS][4] = {
        TQ_GEMM_ROW(TQ_I8, TQ_SCALE_TENSOR, 4, 4, 4, 4, 64, 2),
        TQ_GEMM_ROW(TQ_I8, TQ_SCALE_GROUP_F16, 4, 4, 4, 4, 64, 2),
        TQ_GEMM_NONE,    // groups of 16 are below the 64-column int8 step
        TQ_GEMM_NONE,
        TQ_GEMM_NONE,    // the compact base-3 codec takes bf16 activations
    };
    return t;
}
