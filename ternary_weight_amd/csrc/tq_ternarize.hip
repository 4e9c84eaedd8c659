// libtq: tq_ternarize -- fit a dense weight into K trit planes with scales,
// or into the balanced-ternary codec (the step before tq_pack).
//
// What is computed is stated in tq.h: each matrix is fit on its own into a
// sum of K per-group-scaled trit-planes, weight-only (sasori page, "How it
// works & paper"), plane by plane on the residual; the d = 3 codec is a
// uniform quantisation onto 27 levels with a log-spaced scale codebook,
// groups of 16 (d3 card, "Quantization details").
//
// Mapping onto CDNA4.  One thread owns one group of one row (or, for a
// per-tensor scale, one row) and walks its inputs in index order: the sums
// that set a scale are then the same fp64 additions in the same order as
// the CPU oracle's, so every scale and every trit comes out bit for bit
// equal.  The residual of plane k is not stored: it is replayed from the
// weight and the planes already written, R = fl(...fl(fl(w - s0 t0) - s1 t1)...),
// the same fp32 operations in the same order.  The fit is an offline step
// (a weight is read 2K + 1 times); the loads of neighbouring threads are a
// group apart and each thread's walk reuses its cache lines.
#include <string.h>

#include <cmath>
#include <mutex>
#include <vector>

#include "tq_internal.h"
#include "tq_decode.h"

namespace {

using tqk::f16_to_f32;

// fp32 -> binary16 bits, round to nearest even; finite values above the
// largest half saturate to it (written out so that it is the same rounding
// whatever the mode register says about f16 denormals).
__device__ __forceinline__ uint16_t f32_to_f16_rne(float f)
{
    const uint32_t x = __float_as_uint(f);
    const uint32_t sign = (x >> 16) & 0x8000u;
    const uint32_t ax = x & 0x7FFFFFFFu;
    if (ax >= 0x477FF000u) return (uint16_t)(sign | 0x7BFFu);   // rounds to >= 65520 or is huge
    if (ax < 0x33000001u) return (uint16_t)sign;                // |f| <= 2^-25: zero (ties to even)
    int e = (int)(ax >> 23) - 127;
    uint32_t m = (ax & 0x7FFFFFu) | 0x800000u;                  // 24-bit significand
    if (e < -14) {   // subnormal half: f = m 2^(e-23) = (m >> (-e-1)) 2^-24 plus the remainder
        const int sh = -1 - e;                                  // 14 .. 24
        const uint32_t q = sh < 32 ? m >> sh : 0u;
        const uint32_t rem = m & ((1u << sh) - 1u), half = 1u << (sh - 1);
        const uint32_t r = q + ((rem > half || (rem == half && (q & 1u))) ? 1u : 0u);
        return (uint16_t)(sign | r);
    }
    uint32_t q = m >> 13, rem = m & 0x1FFFu;
    q += (rem > 0x1000u || (rem == 0x1000u && (q & 1u))) ? 1u : 0u;   // may carry into 2^11
    uint32_t exp = (uint32_t)(e + 15);
    if (q == 0x800u) {
        q = 0x400u;
        exp += 1;
    }
    if (exp >= 31) return (uint16_t)(sign | 0x7BFFu);
    return (uint16_t)(sign | (exp << 10) | (q & 0x3FFu));
}

// The plane's trit of residual r: sign(r) where |r| > a / 2 (a > 0), else 0.
__device__ __forceinline__ float trit_of(float r, float a)
{
    return (a > 0.0f && fabsf(r) > 0.5f * a) ? (r > 0.0f ? 1.0f : -1.0f) : 0.0f;
}

// The residual of plane k at input i of a walk: the weight with the planes
// 0 .. k-1 taken off, fp32, one subtraction per plane in plane order.
__device__ __forceinline__ float replay(float w, const int8_t* t, int64_t plane_stride, const float* s, int k)
{
    float r = w;
    for (int kk = 0; kk < k; ++kk) r = __fsub_rn(r, __fmul_rn(s[kk], (float)t[kk * plane_stride]));
    return r;
}

// One lane per (row, group), 64 consecutive groups per workgroup (in the
// flattened (row, group) order they are one contiguous run of the weight):
// the run is loaded into LDS with 16-byte loads, each lane then walks its
// group's residual there (row stride g + 1 floats, so the 64 lanes of a
// read fall in distinct banks), updating it in place plane by plane, and
// writes its trits four to a dword.
constexpr int kTernLanes = 64;

__global__ __launch_bounds__(kTernLanes) void k_tern_group_lds(const float* __restrict__ w, int64_t N, int64_t Kin,
                                                              int g, int K, int8_t* __restrict__ trits,
                                                              uint16_t* __restrict__ scales)
{
    extern __shared__ float R[];                     // [64][g + 1]
    const int64_t G = Kin / g, total = N * G;
    const int64_t id0 = (int64_t)blockIdx.x * kTernLanes;
    const int lane = threadIdx.x;
    const int ngr = (int)(total - id0 < kTernLanes ? total - id0 : kTernLanes);
    // load the run: ngr * g floats from w + id0 * g (g is a multiple of 16)
    const float4* src = (const float4*)(w + id0 * g);
    const int n4 = ngr * g / 4;
    for (int v = lane; v < n4; v += kTernLanes) {
        const float4 x = src[v];
        const int e = v * 4, grp = e / g, i = e - grp * g;
        float* row = R + grp * (g + 1) + i;
        row[0] = x.x;
        row[1] = x.y;
        row[2] = x.z;
        row[3] = x.w;
    }
    __syncthreads();
    if (lane >= ngr) return;
    const int64_t id = id0 + lane;
    float* r = R + lane * (g + 1);
    const int64_t ps = N * Kin;
    uint32_t* tw = (uint32_t*)(trits + id * g);      // the group's trits of plane 0, 4-byte aligned (g % 16 == 0)
    double sum = 0.0;                                  // plane 0's sum of |R|
    for (int i = 0; i < g; ++i) sum += fabs((double)r[i]);
    for (int k = 0; k < K; ++k) {
        const float a = (float)(sum / (double)g);
        double sum_nz = 0.0;
        int64_t nz = 0;
        for (int i = 0; i < g; ++i) {
            if (trit_of(r[i], a) != 0.0f) {
                sum_nz += fabs((double)r[i]);
                nz += 1;
            }
        }
        const float sc = nz > 0 ? (float)(sum_nz / (double)nz) : 0.0f;
        const uint16_t h = f32_to_f16_rne(sc);
        scales[(int64_t)k * total + id] = h;
        const float sv = f16_to_f32(h);
        // write the trits, take the plane off the residual, and sum the next
        // plane's |R| in the same index order
        uint32_t* twk = (uint32_t*)((int8_t*)tw + (int64_t)k * ps);
        sum = 0.0;
        for (int i = 0; i < g; i += 4) {
            uint32_t word = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float t = trit_of(r[i + b], a);
                const float nr = __fsub_rn(r[i + b], __fmul_rn(sv, t));
                r[i + b] = nr;
                sum += fabs((double)nr);
                word |= (uint32_t)(uint8_t)(int8_t)t << (8 * b);
            }
            twk[i / 4] = word;
        }
    }
}

// One thread per (row, group): the K greedy planes of the group (groups
// too long for the LDS walk).
__global__ void k_tern_group(const float* __restrict__ w, int64_t N, int64_t Kin, int g, int K,
                             int8_t* __restrict__ trits, uint16_t* __restrict__ scales)
{
    const int64_t G = Kin / g;
    const int64_t id = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (id >= N * G) return;
    const int64_t n = id / G, j = id - n * G;
    const float* wr = w + n * Kin + j * g;
    const int64_t ps = N * Kin;                      // plane stride of trits
    int8_t* tr = trits + n * Kin + j * g;
    float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int k = 0; k < K; ++k) {
        double sum = 0.0;
        for (int i = 0; i < g; ++i) sum += fabs((double)replay(wr[i], tr + i, ps, s, k));
        const float a = (float)(sum / (double)g);
        double sum_nz = 0.0;
        int64_t nz = 0;
        for (int i = 0; i < g; ++i) {
            const float r = replay(wr[i], tr + i, ps, s, k);
            const float t = trit_of(r, a);
            tr[k * ps + i] = (int8_t)t;
            if (t != 0.0f) {
                sum_nz += fabs((double)r);
                nz += 1;
            }
        }
        const float sc = nz > 0 ? (float)(sum_nz / (double)nz) : 0.0f;
        const uint16_t h = f32_to_f16_rne(sc);
        scales[((int64_t)k * N + n) * G + j] = h;
        s[k] = f16_to_f32(h);
    }
}

// Per-tensor scale, one plane at a time.  Pass 0: per row, sum |R| (fp64,
// index order).  Pass 1: per row, the trits from the absmean a and the sum
// and count of |R| where t != 0.
__global__ void k_tern_rows(const float* __restrict__ w, int64_t N, int64_t Kin, int k, int pass,
                            int8_t* __restrict__ trits, const float* __restrict__ plane_scales,
                            const float* __restrict__ absmean, double* __restrict__ rowsum,
                            int64_t* __restrict__ rownz)
{
    const int64_t n = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (n >= N) return;
    float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int kk = 0; kk < k; ++kk) s[kk] = plane_scales[kk];
    const float* wr = w + n * Kin;
    const int64_t ps = N * Kin;
    int8_t* tr = trits + n * Kin;
    double sum = 0.0;
    int64_t nz = 0;
    const float a = pass == 1 ? *absmean : 0.0f;
    for (int64_t i = 0; i < Kin; ++i) {
        const float r = replay(wr[i], tr + i, ps, s, k);
        if (pass == 0) {
            sum += fabs((double)r);
        } else {
            const float t = trit_of(r, a);
            tr[k * ps + i] = (int8_t)t;
            if (t != 0.0f) {
                sum += fabs((double)r);
                nz += 1;
            }
        }
    }
    rowsum[n] = sum;
    if (pass == 1) rownz[n] = nz;
}

// One thread: the row sums added in row order.  Pass 0: the absmean of the
// plane's residual; pass 1: its least-squares scale (written to scales[k]).
__global__ void k_tern_reduce(int64_t N, int64_t Kin, int k, int pass, const double* __restrict__ rowsum,
                              const int64_t* __restrict__ rownz, float* __restrict__ absmean,
                              float* __restrict__ scales)
{
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    double tot = 0.0;
    int64_t nz = 0;
    for (int64_t n = 0; n < N; ++n) tot += rowsum[n];
    if (pass == 0) {
        *absmean = N * Kin > 0 ? (float)(tot / (double)(N * Kin)) : 0.0f;
        return;
    }
    for (int64_t n = 0; n < N; ++n) nz += rownz[n];
    scales[k] = nz > 0 ? (float)(tot / (double)nz) : 0.0f;
}

// The codec: one thread per (row, group): the smallest codebook entry that
// covers max|w| / L, then L-level uniform quantisation and balanced-ternary
// digits, plane p holding the digit of 3^(K-1-p).
__global__ void k_tern_codec(const float* __restrict__ w, int64_t N, int64_t Kin, int g, int K, int L,
                             const uint16_t* __restrict__ cb, int n_cb, int8_t* __restrict__ trits,
                             uint8_t* __restrict__ idx_out)
{
    __shared__ float cbf[32];
    if (threadIdx.x < 32) cbf[threadIdx.x] = threadIdx.x < (unsigned)n_cb ? f16_to_f32(cb[threadIdx.x]) : 0.0f;
    __syncthreads();
    const int64_t G = Kin / g;
    const int64_t id = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (id >= N * G) return;
    const int64_t n = id / G, j = id - n * G;
    const float* wr = w + n * Kin + j * g;
    float a = 0.0f;
    for (int i = 0; i < g; ++i) a = fmaxf(a, fabsf(wr[i]));
    const float c = __fdiv_rn(a, (float)L);
    int idx = n_cb - 1;
    for (int e = 0; e < n_cb; ++e) {
        if (cbf[e] >= c) {
            idx = e;
            break;
        }
    }
    idx_out[n * G + j] = (uint8_t)idx;
    const float s = cbf[idx];
    const int64_t ps = N * Kin;
    for (int i = 0; i < g; ++i) {
        const float qf = fminf(fmaxf(rintf(__fdiv_rn(wr[i], s)), -(float)L), (float)L);
        int q = (int)qf;
        for (int d = 0; d < K; ++d) {   // digit d (weight 3^d) goes to plane K-1-d
            const int r = ((q % 3) + 3) % 3;
            const int t = r == 2 ? -1 : r;
            trits[(int64_t)(K - 1 - d) * ps + n * Kin + j * g + i] = (int8_t)t;
            q = (q - t) / 3;
        }
    }
}

size_t tensor_ws_bytes(int64_t N) { return (size_t)(N * 16 + 256); }

// Scratch of tq_ternarize_noalloc: the per-row sums, counts and the absmean
// of the per-tensor fit, for up to kNoallocRows rows.  Each GPU the library
// runs on holds its own copy until the process ends.  In host code the name
// is only a stand-in; the device address comes from hipGetSymbolAddress.
constexpr int64_t kNoallocRows = 1 << 18;
constexpr size_t kScratchBytes = (size_t)kNoallocRows * 16 + 256;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up on the first call
// on that device (with it current) and kept.
tq_status scratch_of_current_device(void** out)
{
    int dev = -1;
    tq_status s;
    if ((s = tq_check_hip(hipGetDevice(&dev), "tq_ternarize_noalloc device"))) return s;
    if (dev < 0 || dev >= kMaxDevices) return tq_fail(TQ_ERR_DEVICE, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if ((s = tq_check_hip(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "tq_ternarize_noalloc scratch address")))
            return s;
        if (!p) return tq_fail(TQ_ERR_DEVICE, "tq_ternarize_noalloc: no device address for the scratch array");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return TQ_OK;
}

}  // namespace

TQ_EXPORT tq_status tq_ternarize_workspace_size(const tq_weight_desc* desc, size_t* bytes)
{
    if (!bytes) return tq_fail(TQ_ERR_ARG, "bytes is NULL");
    tq_layout L;
    tq_status s = tq_check_desc(desc, &L);
    if (s) return s;
    *bytes = L.layout == TQ_SCALE_TENSOR ? tensor_ws_bytes(L.N) : 0;
    return tq_ok();
}

TQ_EXPORT tq_status tq_ternarize(const tq_weight_desc* desc, const float* w, const uint16_t* codebook,
                                 int8_t* trits, void* scales, void* workspace, size_t workspace_bytes,
                                 void* stream)
{
    tq_layout L;
    tq_status s = tq_check_desc(desc, &L);
    if (s) return s;
    if ((s = tq_check_ptr(w, "w", false, 4))) return s;
    if ((s = tq_check_ptr(trits, "trits", false, 1))) return s;
    if ((s = tq_check_ptr(scales, "scales", false, L.layout == TQ_SCALE_TENSOR ? 4 : (L.layout == TQ_SCALE_GROUP_F16 ? 2 : 1))))
        return s;
    hipStream_t st = (hipStream_t)stream;
    const int64_t N = L.N, Kin = L.Kin;
    if (N == 0 || Kin == 0) return tq_ok();
    if (tq_is_codebook(L.layout)) {   // the canonical arrays of both codec layouts are alike
        if ((s = tq_check_ptr(codebook, "codebook", false, 2))) return s;
        // the codebook must ascend, from a positive entry: read it back (an offline call)
        uint16_t cb[32];
        if ((s = tq_check_hip(hipMemcpyAsync(cb, codebook, 2 * (size_t)L.ncb, hipMemcpyDeviceToHost, st),
                              "tq_ternarize codebook")))
            return s;
        if ((s = tq_check_hip(hipStreamSynchronize(st), "tq_ternarize synchronize"))) return s;
        float prev = 0.0f;
        for (int e = 0; e < L.ncb; ++e) {
            const float v = (float)__builtin_bit_cast(_Float16, cb[e]);
            if (!(v > prev) || !std::isfinite(v))
                return tq_fail(TQ_ERR_VALUE, "codebook entry %d (%g) is not positive, finite and ascending", e, v);
            prev = v;
        }
        const int Lv = L.K == 1 ? 1 : (L.K == 2 ? 4 : (L.K == 3 ? 13 : 40));
        const int64_t threads = N * (Kin / L.g);
        hipLaunchKernelGGL(k_tern_codec, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, w, N, Kin, L.g,
                           L.K, Lv, codebook, L.ncb, trits, (uint8_t*)scales);
        return tq_check_launch("tq_ternarize") ? TQ_ERR_DEVICE : tq_ok();
    }
    if (L.layout == TQ_SCALE_GROUP_F16) {
        const int64_t groups = N * (Kin / L.g);
        const size_t lds = (size_t)kTernLanes * (L.g + 1) * sizeof(float);
        static bool lds_raised = false;   // the default dynamic-LDS limit is 64 KiB
        if (!lds_raised) {
            lds_raised = hipFuncSetAttribute((const void*)k_tern_group_lds,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, TQ_MAX_WG_LDS) == hipSuccess;
        }
        if ((lds <= 65536 || lds_raised) && lds <= TQ_MAX_WG_LDS && ((uintptr_t)w & 15) == 0 &&
            ((uintptr_t)trits & 3) == 0) {
            hipLaunchKernelGGL(k_tern_group_lds, dim3((unsigned)((groups + kTernLanes - 1) / kTernLanes)),
                               dim3(kTernLanes), lds, st, w, N, Kin, L.g, L.K, trits, (uint16_t*)scales);
        } else {
            hipLaunchKernelGGL(k_tern_group, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, st, w, N, Kin,
                               L.g, L.K, trits, (uint16_t*)scales);
        }
        return tq_check_launch("tq_ternarize") ? TQ_ERR_DEVICE : tq_ok();
    }
    // per-tensor scale: per-row passes and single-thread reductions, plane by plane
    if ((s = tq_check_ptr(workspace, "workspace", false, 256))) return s;
    if (workspace_bytes < tensor_ws_bytes(N))
        return tq_fail(TQ_ERR_ARG, "workspace has %zu bytes, needs %zu", workspace_bytes, tensor_ws_bytes(N));
    double* rowsum = (double*)workspace;
    int64_t* rownz = (int64_t*)((uint8_t*)workspace + 8 * N);
    float* absmean = (float*)((uint8_t*)workspace + 16 * N);
    float* ps = (float*)scales;
    const dim3 grid((unsigned)((N + 255) / 256)), block(256);
    for (int k = 0; k < L.K; ++k) {
        hipLaunchKernelGGL(k_tern_rows, grid, block, 0, st, w, N, Kin, k, 0, trits, ps, absmean, rowsum, rownz);
        hipLaunchKernelGGL(k_tern_reduce, dim3(1), dim3(64), 0, st, N, Kin, k, 0, rowsum, rownz, absmean, ps);
        hipLaunchKernelGGL(k_tern_rows, grid, block, 0, st, w, N, Kin, k, 1, trits, ps, absmean, rowsum, rownz);
        hipLaunchKernelGGL(k_tern_reduce, dim3(1), dim3(64), 0, st, N, Kin, k, 1, rowsum, rownz, absmean, ps);
    }
    return tq_check_launch("tq_ternarize") ? TQ_ERR_DEVICE : tq_ok();
}

TQ_EXPORT tq_status tq_ternarize_noalloc(const tq_weight_desc* desc, const float* w, const uint16_t* codebook,
                                         int8_t* trits, void* scales, void* stream)
{
    tq_layout L;
    tq_status s = tq_check_desc(desc, &L);
    if (s) return s;
    if (L.layout != TQ_SCALE_TENSOR)   // these fits use no scratch
        return tq_ternarize(desc, w, codebook, trits, scales, nullptr, 0, stream);
    if (L.N > kNoallocRows)
        return tq_fail(TQ_ERR_UNSUPPORTED, "tq_ternarize_noalloc: %lld rows exceed the %lld its scratch holds",
                       (long long)L.N, (long long)kNoallocRows);
    void* ws = nullptr;
    if ((s = scratch_of_current_device(&ws))) return s;
    return tq_ternarize(desc, w, codebook, trits, scales, ws, kScratchBytes, stream);
}
