// libtq: bf16-activation prefill kernels (bf16 MFMA, fp32 accumulate).
#include "tq_gemm_impl.h"
#include "tq_gemm_kernels.h"

TQ_GEMM_TABLE(tq_gemm_table_bf16, TQ_BF16, 4, 4, 4, 4)
