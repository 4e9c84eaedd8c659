// libtq: tq_act_quant_int8 -- per-token absmax int8 quantisation.
//
// a = max|x| over the token; inv = fl32(127 / a); q = clamp(rne(fl32(x * inv)),
// -127, 127); s = fl32(a / 127); a zero token gives q = 0 and s = 0.  The
// division and the product are single IEEE fp32 operations (this file is built
// with -ffp-contract=off; HIP divides fp32 with correct rounding), so the
// result is bit-identical to any IEEE implementation of the same steps.
#include <string.h>

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

struct Seg {
    int64_t row0;        // first global row of the segment
    int64_t Kin;
    int32_t x_type, pad;
    const void* x;
    int8_t* q;
    float* s;
};

struct SegTable {
    Seg seg[TQ_ACT_MAX_SEGMENTS];
    int32_t count;
};

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kHeld = 8;   // 16-byte vectors a thread keeps: one pass for Kin <= 8 * 4 * kThreads

__device__ __forceinline__ float absmax4(f32x4 v)
{
    return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

__device__ __forceinline__ uint32_t quant4(f32x4 v, float inv)
{
    return (uint32_t)(uint8_t)quant1(v.x, inv) | ((uint32_t)(uint8_t)quant1(v.y, inv) << 8) |
           ((uint32_t)(uint8_t)quant1(v.z, inv) << 16) | ((uint32_t)(uint8_t)quant1(v.w, inv) << 24);
}

// four values of a row as fp32: fp32 loads 16 bytes, bf16 loads 8 bytes
template <int XT>
__device__ __forceinline__ f32x4 load4(const void* row, int i)
{
    if (XT == TQ_F32) return reinterpret_cast<const f32x4*>(row)[i];
    const uint2 w = reinterpret_cast<const uint2*>(row)[i];
    return f32x4{bf16_to_f32(w.x & 0xFFFFu), bf16_to_f32(w.x >> 16), bf16_to_f32(w.y & 0xFFFFu),
                 bf16_to_f32(w.y >> 16)};
}

// One workgroup per token (row): a = max|x| (each thread keeps its values in
// registers when the row fits), then q and s.  Kin % 16 == 0.
template <int XT>
__device__ __forceinline__ void quant_row(const void* xrow, int8_t* qrow, float* s_out, int64_t Kin)
{
    __shared__ float red[kThreads / 64];
    const int tid = threadIdx.x;
    const int n4 = (int)(Kin >> 2);
    const bool held = n4 <= kHeld * kThreads;
    f32x4 v[kHeld];
    float a = 0.0f;
    if (held) {
#pragma unroll
        for (int j = 0; j < kHeld; ++j) {
            const int i = tid + j * kThreads;
            v[j] = i < n4 ? load4<XT>(xrow, i) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            a = fmaxf(a, absmax4(v[j]));
        }
    } else {
        for (int i = tid; i < n4; i += kThreads) a = fmaxf(a, absmax4(load4<XT>(xrow, i)));
    }
    a = wave_max(a);
    if ((tid & 63) == 0) red[tid >> 6] = a;
    __syncthreads();
    a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float inv = a > 0.0f ? 127.0f / a : 0.0f;
    uint32_t* q4 = reinterpret_cast<uint32_t*>(qrow);
    if (held) {
#pragma unroll
        for (int j = 0; j < kHeld; ++j) {
            const int i = tid + j * kThreads;
            if (i < n4) q4[i] = quant4(v[j], inv);
        }
    } else {
        for (int i = tid; i < n4; i += kThreads) q4[i] = quant4(load4<XT>(xrow, i), inv);
    }
    if (tid == 0) *s_out = a > 0.0f ? a / 127.0f : 0.0f;
}

template <int XT>
__global__ __launch_bounds__(kThreads) void k_act_quant(const void* __restrict__ x, int8_t* __restrict__ q,
                                                        float* __restrict__ s, int64_t Kin)
{
    const int64_t m = blockIdx.x;
    const size_t esz = XT == TQ_F32 ? 4 : 2;
    quant_row<XT>((const uint8_t*)x + m * Kin * esz, q + m * Kin, s + m, Kin);
}

// Several matrices in one launch: workgroup b is global row b.
__global__ __launch_bounds__(kThreads) void k_act_quant_batch(SegTable T)
{
    const int64_t b = blockIdx.x;
    int j = 0;
    while (j + 1 < T.count && T.seg[j + 1].row0 <= b) ++j;
    const Seg& S = T.seg[j];
    const int64_t m = b - S.row0;
    if (S.x_type == TQ_F32)
        quant_row<TQ_F32>((const float*)S.x + m * S.Kin, S.q + m * S.Kin, S.s + m, S.Kin);
    else
        quant_row<TQ_BF16>((const uint16_t*)S.x + m * S.Kin, S.q + m * S.Kin, S.s + m, S.Kin);
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
    if ((s = tq_check_ptr(x_scale, "x_scale", false, 4))) return s;
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

TQ_EXPORT tq_status tq_act_quant_int8_batch(const tq_act_segment* segments, int32_t count, void* stream_)
{
    tq_status s;
    if (count < 0 || count > TQ_ACT_MAX_SEGMENTS || (count > 0 && !segments))
        return tq_fail(TQ_ERR_ARG, "count = %d, must be 0..%d", count, TQ_ACT_MAX_SEGMENTS);
    SegTable T;
    memset(&T, 0, sizeof T);
    int64_t rows = 0;
    for (int32_t i = 0; i < count; ++i) {
        const tq_act_segment& g = segments[i];
        if (g.M < 0 || g.in_features < 0)
            return tq_fail(TQ_ERR_ARG, "segment %d: negative size", i);
        if (g.x_type != TQ_F32 && g.x_type != TQ_BF16)
            return tq_fail(TQ_ERR_ARG, "segment %d: x_type = %d, must be TQ_F32 or TQ_BF16", i, g.x_type);
        if (g.in_features % 16 || g.in_features > TQ_MAX_KIN)
            return tq_fail(TQ_ERR_SHAPE, "segment %d: in_features = %lld", i, (long long)g.in_features);
        if (g.M > 0) {
            const bool need = g.in_features > 0;
            if ((s = tq_check_ptr(g.x, "segment x", !need))) return s;
            if ((s = tq_check_ptr(g.xq, "segment xq", !need))) return s;
            if ((s = tq_check_ptr(g.x_scale, "segment x_scale", false, 4))) return s;
        }
        Seg& d = T.seg[T.count++];
        d.row0 = rows;
        d.Kin = g.in_features;
        d.x_type = g.x_type;
        d.x = g.x;
        d.q = g.xq;
        d.s = g.x_scale;
        rows += g.M;
    }
    if (rows > (1ll << 31) - 1) return tq_fail(TQ_ERR_SHAPE, "too many rows");
    if (rows == 0) return tq_ok();
    hipLaunchKernelGGL(k_act_quant_batch, dim3((unsigned)rows), dim3(kThreads), 0, (hipStream_t)stream_, T);
    if ((s = tq_check_launch("tq_act_quant_int8_batch"))) return s;
    return tq_ok();
}
