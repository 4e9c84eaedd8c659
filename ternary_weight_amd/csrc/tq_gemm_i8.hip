// libtq: int8-activation prefill kernels (int8 MFMA, int32 accumulate).
#include "tq_gemm_impl.h"
#include "tq_gemm_kernels.h"

// one plane, per-tensor scale: 4 x 8 tiles per wave; the rest keep an fp32
// accumulator beside the int32 partial sums, so 4 x 4
TQ_GEMM_TABLE(tq_gemm_table_i8, TQ_I8, 4, 8, 4, 4)
