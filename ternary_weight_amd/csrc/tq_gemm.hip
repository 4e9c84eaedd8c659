// libtq: tq_gemm -- prefill product on the matrix cores (MFMA).
#include "tq_internal.h"

TQ_EXPORT tq_status tq_gemm(const tq_weight_desc* desc, const void* blob, int64_t M, int32_t x_type,
                            const void* x, const float* x_scale, float* y, int32_t* acc, void* stream)
{
    (void)blob; (void)M; (void)x_type; (void)x; (void)x_scale; (void)y; (void)acc; (void)stream;
    tq_layout L;
    tq_status s = tq_check_desc(desc, &L);
    if (s) return s;
    return tq_fail(TQ_ERR_UNSUPPORTED, "tq_gemm: not available in this build");
}
