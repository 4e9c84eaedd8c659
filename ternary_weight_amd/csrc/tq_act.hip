// libtq: tq_act_quant_int8 -- per-token absmax int8 quantisation.
//
// a = max|x| over the token; inv = fl32(127 / a); q = clamp(rne(fl32(x * inv)),
// -127, 127); s = fl32(a / 127); a zero token gives q = 0 and s = 0.  The
// division and the product are single IEEE fp32 operations (this file is built
// with -ffp-contract=off; HIP divides fp32 with correct rounding), so the
// result is bit-identical to any IEEE implementation of the same steps.
#include "tq_internal.h"

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ int8_t quant1(float v, float inv)
{
    float r = rintf(v * inv);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int8_t)(int)r;
}

// One workgroup per token; Kin % 16 == 0 so every row starts 16-byte aligned.
template <int XT>
__global__ __launch_bounds__(kThreads) void k_act_quant(const void* __restrict__ x,
                                                        int8_t* __restrict__ q,
                                                        float* __restrict__ s, int64_t Kin)
{
    __shared__ float red[kThreads / 64];
    const int64_t m = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t n16 = Kin / 16;   // 16-element units
    float a = 0.0f;
    if (XT == TQ_F32) {
        const float4* xr = reinterpret_cast<const float4*>((const float*)x + m * Kin);
        for (int64_t u = tid; u < n16 * 4; u += kThreads) {
            const float4 v = xr[u];
            a = fmaxf(a, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        }
    } else {
        const uint4* xr = reinterpret_cast<const uint4*>((const uint16_t*)x + m * Kin);
        for (int64_t u = tid; u < n16 * 2; u += kThreads) {
            const uint4 v = xr[u];
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                a = fmaxf(a, fabsf(bf16_to_f32(w[j] & 0xFFFFu)));
                a = fmaxf(a, fabsf(bf16_to_f32(w[j] >> 16)));
            }
        }
    }
    a = wave_max(a);
    if ((tid & 63) == 0) red[tid >> 6] = a;
    __syncthreads();
    a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float inv = a > 0.0f ? 127.0f / a : 0.0f;
    int8_t* qr = q + m * Kin;
    if (XT == TQ_F32) {
        const float4* xr = reinterpret_cast<const float4*>((const float*)x + m * Kin);
        for (int64_t u = tid; u < n16 * 4; u += kThreads) {
            const float4 v = xr[u];
            const uint32_t b = (uint32_t)(uint8_t)quant1(v.x, inv) |
                               ((uint32_t)(uint8_t)quant1(v.y, inv) << 8) |
                               ((uint32_t)(uint8_t)quant1(v.z, inv) << 16) |
                               ((uint32_t)(uint8_t)quant1(v.w, inv) << 24);
            reinterpret_cast<uint32_t*>(qr)[u] = b;
        }
    } else {
        const uint4* xr = reinterpret_cast<const uint4*>((const uint16_t*)x + m * Kin);
        for (int64_t u = tid; u < n16 * 2; u += kThreads) {
            const uint4 v = xr[u];
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
            uint32_t o[2] = {0, 0};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t lo = (uint8_t)quant1(bf16_to_f32(w[j] & 0xFFFFu), inv);
                const uint32_t hi = (uint8_t)quant1(bf16_to_f32(w[j] >> 16), inv);
                o[j >> 1] |= (lo | (hi << 8)) << (16 * (j & 1));
            }
            reinterpret_cast<uint2*>(qr)[u] = make_uint2(o[0], o[1]);
        }
    }
    if (tid == 0) s[m] = a > 0.0f ? a / 127.0f : 0.0f;
}

}  // namespace

TQ_EXPORT tq_status tq_act_quant_int8(int64_t M, int64_t Kin, int32_t x_type, const void* x,
                                      int8_t* xq, float* x_scale, void* stream_)
{
    tq_status s;
    if (M < 0 || Kin < 0) return tq_fail(TQ_ERR_ARG, "negative size M = %lld, Kin = %lld",
                                         (long long)M, (long long)Kin);
    if (x_type != TQ_F32 && x_type != TQ_BF16)
        return tq_fail(TQ_ERR_ARG, "x_type = %d, must be TQ_F32 or TQ_BF16", x_type);
    if (Kin % 16) return tq_fail(TQ_ERR_SHAPE, "in_features = %lld is not a multiple of 16",
                                 (long long)Kin);
    if (Kin > TQ_MAX_KIN || M > (1ll << 31) - 1)
        return tq_fail(TQ_ERR_SHAPE, "M = %lld, Kin = %lld out of range", (long long)M,
                       (long long)Kin);
    if (M == 0) return tq_ok();
    const bool need = Kin > 0;
    if ((s = tq_check_ptr(x, "x", !need))) return s;
    if ((s = tq_check_ptr(xq, "xq", !need))) return s;
    if ((s = tq_check_ptr(x_scale, "x_scale", false))) return s;
    hipStream_t stream = (hipStream_t)stream_;
    if (x_type == TQ_F32)
        hipLaunchKernelGGL(k_act_quant<TQ_F32>, dim3((unsigned)M), dim3(kThreads), 0, stream, x, xq,
                           x_scale, Kin);
    else
        hipLaunchKernelGGL(k_act_quant<TQ_BF16>, dim3((unsigned)M), dim3(kThreads), 0, stream, x,
                           xq, x_scale, Kin);
    if ((s = tq_check_launch("tq_act_quant_int8"))) return s;
    return tq_ok();
}
