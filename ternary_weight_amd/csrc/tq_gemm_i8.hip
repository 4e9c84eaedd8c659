// libtq: int8-activation prefill kernels (int8 MFMA, int32 accumulate).
#include "tq_gemm_impl.h"
#include "tq_gemm_kernels.h"

// One plane with a per-tensor scale (the int32 sums are the result, no
// scaled partial sums to keep): 4 x 8 tiles per wave, a 128-token x 256-row
// workgroup tile, at two waves per SIMD (211 VGPRs); the workgroup stages each
// row's whole 16-byte code slot per step, one row per thread, and every
// barrier covers 32 MFMAs per wave.  BitNet-2B-shaped stack at 2048 tokens:
// 5.06 -> 4.33 ms against 4 x 4 tiles; 8 x 8 tiles at one wave per SIMD and
// two steps in flight instead of four were slower.  The layouts with group
// scales keep 4 x 4 tiles: their scaled sums need a second set of
// accumulators, which 4 x 8 tiles cannot hold at two waves per SIMD.
const tq_gemm_kernel (*tq_gemm_table_i8())[4]
{
    static const tq_gemm_kernel t[TQ_GEMM_ROWS][4] = {
        TQ_GEMM_ROW(TQ_I8, TQ_SCALE_TENSOR, 4, 8, 4, 4, 64, 2),
        TQ_GEMM_ROW(TQ_I8, TQ_SCALE_GROUP_F16, 4, 4, 4, 4, 64, 2),
        TQ_GEMM_NONE,    // groups of 16 are below the 64-column int8 step
        TQ_GEMM_NONE,
        TQ_GEMM_NONE,    // the compact base-3 codec takes bf16 activations
    };
    return t;
}
