// libtq: int8-activation prefill kernels (int8 MFMA, int32 accumulate).
#include "tq_gemm_impl.h"
#include "tq_gemm_kernels.h"

// One plane with a per-tensor scale keeps only int32 sums: 4 x 8 tiles per
// wave.  The rest keep an fp32 accumulator beside them: 4 x 4.
const tq_gemm_kernel (*tq_gemm_table_i8())[4]
{
    static const tq_gemm_kernel t[TQ_GEMM_ROWS][4] = {
        TQ_GEMM_ROW(TQ_I8, TQ_SCALE_TENSOR, 4, 8, 4, 4, 64, 2),
        TQ_GEMM_ROW(TQ_I8, TQ_SCALE_GROUP_F16, 4, 4, 4, 4, 64, 2),
        TQ_GEMM_NONE,    // groups of 16 are below the 64-column int8 step
        TQ_GEMM_NONE,
    };
    return t;
}
