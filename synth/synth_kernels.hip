// Device copy of the seeded input generator (synth/gen.py) -- test and
// benchmark infrastructure, not part of libtq.
//
// Each element is computed from its index alone (SplitMix64 is counter based:
// output i of seed s is mix64(s + (i+1) * GAMMA)), and every floating-point
// step is the same IEEE basic operation, in the same order, as in gen.py.
// Built with -ffp-contract=off so no multiply-add is fused; fp64 division is
// correctly rounded.  The only rounding not written out in gen.py is fp64 ->
// f16, done here with exact scaling and rint (round to nearest even), the
// same result numpy's float16 conversion gives.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define SYNTH_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr uint64_t GAMMA = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t draw(uint64_t seed, int64_t i) { return mix64(seed + (uint64_t)(i + 1) * GAMMA); }
__device__ __forceinline__ double u01(uint64_t r) { return (double)(r >> 11) * 0x1.0p-53; }

__device__ __forceinline__ double as_f64(uint64_t b) { return __longlong_as_double((long long)b); }
__device__ __forceinline__ uint64_t as_u64(double d) { return (uint64_t)__double_as_longlong(d); }

constexpr double LN2 = 0x1.62e42fefa39efp-1;
constexpr double LN2_HI = 0x1.62e42fee00000p-1;
constexpr double LN2_LO = 0x1.a39ef35793c76p-33;
constexpr double INV_LN2 = 0x1.71547652b82fep+0;
constexpr double SQRT2 = 0x1.6a09e667f3bcdp+0;
constexpr double HALF_PI = 0x1.921fb54442d18p+0;
constexpr int N_LN = 14, N_TRIG = 14, N_EXP = 22, N_SQRT = 7;

struct Coeffs {
    double ln[N_LN], cs[N_TRIG], sn[N_TRIG], ex[N_EXP];
};

// The series coefficients, computed by the same recurrences as gen.py.
__device__ __forceinline__ void make_coeffs(Coeffs& c)
{
    for (int k = 0; k < N_LN; ++k) c.ln[k] = 1.0 / (double)(2 * k + 1);
    c.cs[0] = 1.0;
    c.sn[0] = 1.0;
    for (int k = 1; k < N_TRIG; ++k) {
        c.cs[k] = c.cs[k - 1] / (-(double)((2 * k - 1) * (2 * k)));
        c.sn[k] = c.sn[k - 1] / (-(double)((2 * k) * (2 * k + 1)));
    }
    c.ex[0] = 1.0;
    for (int k = 1; k < N_EXP; ++k) c.ex[k] = c.ex[k - 1] / (double)k;
}

__device__ double det_ln(double u, const Coeffs& C)
{
    const uint64_t bits = as_u64(u);
    int64_t e = (int64_t)((bits >> 52) & 0x7FF) - 1023;
    double m = as_f64((bits & 0x000FFFFFFFFFFFFFull) | 0x3FF0000000000000ull);
    if (m > SQRT2) {
        m = m * 0.5;
        e = e + 1;
    }
    const double s = (m - 1.0) / (m + 1.0);
    const double s2 = s * s;
    double p = C.ln[N_LN - 1];
    for (int k = N_LN - 2; k >= 0; --k) p = p * s2 + C.ln[k];
    return (double)e * LN2 + (2.0 * s) * p;
}

__device__ double det_cos2pi(double u, const Coeffs& C)
{
    const double v = u * 4.0;
    const double q = floor(v);
    const double f = v - q;
    const bool flip = f > 0.5;
    const double g = flip ? 1.0 - f : f;
    const double x = g * HALF_PI;
    const double x2 = x * x;
    double c = C.cs[N_TRIG - 1];
    for (int k = N_TRIG - 2; k >= 0; --k) c = c * x2 + C.cs[k];
    double s = C.sn[N_TRIG - 1];
    for (int k = N_TRIG - 2; k >= 0; --k) s = s * x2 + C.sn[k];
    s = s * x;
    const double cf = flip ? s : c;
    const double sf = flip ? c : s;
    const int qi = (int)q;
    return qi == 0 ? cf : (qi == 1 ? -sf : (qi == 2 ? -cf : sf));
}

__device__ double det_sqrt(double y)
{
    if (!(y > 0.0)) return 0.0;
    const uint64_t bits = as_u64(y);
    const int64_t e = (int64_t)((bits >> 52) & 0x7FF) - 1023;
    // floor division by 2, as Python's // does
    const int64_t h = (e + 2 >= 0) ? (e + 2) / 2 : -((-(e + 2) + 1) / 2);
    double x = as_f64((uint64_t)(h + 1023) << 52);
    for (int i = 0; i < N_SQRT; ++i) x = 0.5 * (x + y / x);
    return x;
}

__device__ double det_exp(double z, const Coeffs& C)
{
    const double k = floor(z * INV_LN2 + 0.5);
    const double r = (z - k * LN2_HI) - k * LN2_LO;
    double p = C.ex[N_EXP - 1];
    for (int j = N_EXP - 2; j >= 0; --j) p = p * r + C.ex[j];
    const double scale = as_f64((uint64_t)((int64_t)k + 1023) << 52);
    return p * scale;
}

__device__ double normal_at(uint64_t seed, int64_t i, const Coeffs& C)
{
    const double ua = u01(draw(seed, 2 * i));
    const double ub = u01(draw(seed, 2 * i + 1));
    const double rad = det_sqrt(-2.0 * det_ln(1.0 - ua, C));
    return rad * det_cos2pi(ub, C);
}

// fp64 -> IEEE binary16 bits, round to nearest even (finite, |v| < 65520 here).
__device__ uint16_t f64_to_f16(double v)
{
    const uint16_t sign = (as_u64(v) >> 63) ? 0x8000 : 0;
    double a = fabs(v);
    if (a >= 65520.0) return sign | 0x7C00;
    int e = (int)((as_u64(a) >> 52) & 0x7FF) - 1023;
    if (e < -14) {   // subnormal range: units of 2^-24
        const double q = rint(a * 0x1.0p24);
        return sign | (uint16_t)q;   // q == 1024 is the smallest normal, encoded the same way
    }
    // a = q * 2^(e-10) with q in [1024, 2048]
    double q = rint(a * as_f64((uint64_t)(1023 + 10 - e) << 52));
    if (q >= 2048.0) {
        q = q * 0.5;
        e += 1;
    }
    if (e > 15) return sign | 0x7C00;
    return sign | (uint16_t)(((e + 15) << 10) | ((int)q - 1024));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    const uint32_t u = __float_as_uint(f);
    const uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

enum { K_TRITS = 0, K_DIGITS = 1, K_INDICES = 2, K_NORMAL_F32 = 3, K_NORMAL_BF16 = 4,
       K_LOGU_F16 = 5, K_LOGU_F32 = 6, K_NORMAL_F64 = 7 };

__global__ void k_fill(int kind, uint64_t seed, int64_t start, int64_t count, double a, double b,
                       double div, void* out)
{
    Coeffs C;
    make_coeffs(C);
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < count;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = start + t;
        switch (kind) {
        case K_TRITS: {
            const double u = u01(draw(seed, i));
            ((int8_t*)out)[t] = u < 0.3 ? -1 : (u < 0.6 ? 1 : 0);
            break;
        }
        case K_DIGITS: {
            const double u = u01(draw(seed, i));
            ((int8_t*)out)[t] = (int8_t)((int)floor(u * 3.0) - 1);
            break;
        }
        case K_INDICES: {
            const double u = u01(draw(seed, i));
            ((uint8_t*)out)[t] = (uint8_t)(int)floor(u * a);
            break;
        }
        case K_NORMAL_F32:
            ((float*)out)[t] = (float)normal_at(seed, i, C);
            break;
        case K_NORMAL_BF16:
            ((uint16_t*)out)[t] = f32_to_bf16((float)normal_at(seed, i, C));
            break;
        case K_NORMAL_F64:
            ((double*)out)[t] = normal_at(seed, i, C);
            break;
        case K_LOGU_F16: {
            const double u = u01(draw(seed, i));
            ((uint16_t*)out)[t] = f64_to_f16(det_exp(a + u * b, C) / div);
            break;
        }
        case K_LOGU_F32: {
            const double u = u01(draw(seed, i));
            ((float*)out)[t] = (float)(det_exp(a + u * b, C) / div);
            break;
        }
        default:
            break;
        }
    }
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Plain streaming read of n16 16-byte vectors (a bandwidth reference for the
// benchmark): every byte is loaded once, folded by XOR, and the fold is
// stored only under a condition that keeps the loads live.
__global__ void k_stream_read(const u32x4* __restrict__ p, int64_t n16, uint32_t* out)
{
    uint32_t acc = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(p + i);
        const u32x4 b = __builtin_nontemporal_load(p + i + stride);
        const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(p + i + 3 * stride);
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n16; i += stride) {
        const u32x4 a = __builtin_nontemporal_load(p + i);
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == 0x9E3779B9u) out[0] = acc;
}

}  // namespace

// Read `bytes` (a multiple of 16) from a 16-byte aligned device buffer once;
// `out` is a device uint32 that is written only in a practically impossible
// case.  Returns 0 or a hipError_t value.
SYNTH_EXPORT int synth_stream_read(const void* p, int64_t bytes, uint32_t* out, int blocks, void* stream)
{
    if (bytes < 16) return 0;
    hipLaunchKernelGGL(k_stream_read, dim3(blocks > 0 ? blocks : 4096), dim3(256), 0, (hipStream_t)stream,
                       (const u32x4*)p, bytes / 16, out);
    return (int)hipGetLastError();
}

// Fill out[0 .. count) with elements start .. start+count-1 of a stream.
//   kind 0 trits int8, 1 digits int8, 2 indices uint8 (a = n), 3 normal fp32,
//   4 normal bf16 bits, 5 log-uniform f16 bits (a = ln lo, b = ln hi - ln lo,
//   value divided by div), 6 log-uniform fp32 (same), 7 normal fp64.
// Returns 0 on success, else a hipError_t value.
SYNTH_EXPORT int synth_fill(int kind, uint64_t seed, int64_t start, int64_t count, double a,
                            double b, double div, void* out, void* stream)
{
    if (count <= 0) return 0;
    int64_t blocks = (count + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(k_fill, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, kind, seed,
                       start, count, a, b, div, out);
    return (int)hipGetLastError();
}
