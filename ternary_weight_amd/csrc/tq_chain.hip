// libtq: tq_bitnet_chain_* -- BitNet b1.58 layers run back to back for one
// token in one persistent launch (the decode chain).
//
// What a layer computes, step by step, is stated in tq.h; it follows the
// QORA-LLM-2B page's "SubLN Pattern" listing, and its ternary linears are
// the int8-activation product of the decode kernels (one plane, per-tensor
// scale, the exact int32 sum and fl(float(acc) * fl(s_w * s_x))).
//
// Mapping onto CDNA4.  A layer has four phases, each a set of ternary
// linears sharing one input vector:
//   QKV   q, k, v of RMSNorm(x)              -> qkv
//   O     o of RMSNorm(repeat(v))            -> x1 = x + .
//   GU    gate and up of RMSNorm(x1)         -> act = relu2(gate) * up
//   DOWN  down of RMSNorm(act)               -> x = x1 + .
// A phase needs the whole of the vector it normalises (a norm is a
// reduction over it), so it waits until every output block of the phase it
// reads has been written: each block's last writer counts it in a per-layer
// counter once its stores are complete.  O needs only v, so the QKV phase
// produces v first and O starts while q and k are still being computed.
// The launch is cooperative (all workgroups resident; every wait is on
// blocks of an earlier phase, so none can be circular) and each workgroup,
// for each phase in which it has an item:
//   1. issues the code loads of its first item -- weights do not depend on
//      the activations, so they stream in while the workgroup waits;
//   2. waits for the blocks it reads;
//   3. reads the phase's input vector (a few KiB, from L2/HBM, all loads in
//      flight together), takes its RMSNorm and int8 quantisation into LDS --
//      every workgroup does this itself, in the same order, so all hold the
//      same bytes and no extra barrier is needed;
//   4. runs its items: a 64-row block of one projection (GU: the same block
//      of gate and of up, half the waves each), restricted to one of S
//      column splits, the waves splitting that range further (the decode
//      kernels' row-block loop, one row per lane).  The waves' partial sums
//      meet in LDS; with S > 1 the splits of a block meet in an int32
//      accumulator in global memory (exact, any order) and the last split
//      to arrive, counted with an atomic per block, applies the epilogue,
//      clears the accumulator and the count, and counts the block done.
#include <string.h>

#include <algorithm>
#include <cmath>
#include <vector>

#include "tq_gemv_impl.h"

namespace {

using namespace tqk;

#ifndef TQ_CHAIN_THREADS
#define TQ_CHAIN_THREADS 512
#endif
constexpr int kThreads = TQ_CHAIN_THREADS;   // 8 waves (measured against 16)
constexpr int kWaves = kThreads / 64;
constexpr int kMaxWidth = 8192;          // longest phase input (held in registers, 16 per thread)
constexpr uint32_t kSpinLimit = 1u << 22;   // polls of one wait before giving up (~seconds)
#ifndef TQ_CHAIN_SLEEP
#define TQ_CHAIN_SLEEP 16                    // s_sleep between two polls of a wait (units of 64 cycles)
#endif

enum { PH_QKV = 0, PH_O = 1, PH_GU = 2, PH_DOWN = 3 };
enum { W_Q = 0, W_K, W_V, W_O, W_GATE, W_UP, W_DOWN };

struct LayerDev {
    tq_prob_dev p[7];
    const float* norm[4];
};

struct PhaseDev {
    int32_t groups;     // output blocks: 64-row blocks (QKV over q|k|v; GU: gate/up pairs)
    int32_t splits;     // column splits per block
    int32_t items;      // groups * splits
    int32_t width;      // input length
    int32_t acc_base;   // first accumulator row of the phase's blocks
    int32_t cnt_base;   // first arrival counter of the phase's blocks
};

struct ChainDev {
    PhaseDev ph[4];
    int32_t n_layers, hidden, inter, n_heads, n_kv, head_dim;
    int32_t nq, nkv, nb_q, nb_kv, G;
    float eps;
    const LayerDev* layers;
    float* qkv;         // [nq + 2 nkv]
    float* x1;          // [hidden]
    float* act;         // [inter]
    int32_t* acc;       // split partial sums, 64 rows per block, kept zero (sizes_of)
    uint32_t* cnt;      // arrivals per block, kept zero
    uint32_t* done;     // [n_layers][5] blocks written: QKV, v, O, GU, DOWN
    int32_t* err;       // set when a wait gives up
};

// ---------------------------------------------------------------------------
// Device side.
//
// Data that one workgroup writes and others read (the phase outputs and the
// hidden state) moves only through agent-scope accesses, which reach memory
// past the per-XCD L2s (sc1): so no cache needs writing back or invalidating
// at a barrier -- a barrier only waits for the workgroup's own stores to
// complete before it arrives.  Everything else the kernel reads is
// read-only for the whole launch and stays cached.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float ld_shared(const float* p)
{
    return __uint_as_float(__hip_atomic_load((const uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void st_shared(float* p, float v)
{
    __hip_atomic_store((uint32_t*)p, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wave's stores and atomics have completed.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

struct Item {
    int proj;           // projection of waves 0 .. kWaves/2 - 1 (GU) or of all waves
    int rb;             // 64-row block within the projection
    int split;
    int group;
    int off;            // first output row of the block (in q|k|v for QKV)
    int arow;           // first accumulator row of the block (of gate for GU): 64 rows
                        // of its own, apart from every other block that can be in flight
};

__device__ __forceinline__ Item item_of(const ChainDev& C, const PhaseDev& P, int ph, int item)
{
    Item it;
    it.group = item / P.splits;
    it.split = item - it.group * P.splits;
    if (ph == PH_QKV) {   // v first (O waits for it alone), then k, then q
        int g = it.group;
        if (g < C.nb_kv) {
            it.proj = W_V; it.rb = g; it.off = C.nq + C.nkv + g * 64;
        } else if (g < 2 * C.nb_kv) {
            it.proj = W_K; it.rb = g - C.nb_kv; it.off = C.nq + it.rb * 64;
        } else {
            it.proj = W_Q; it.rb = g - 2 * C.nb_kv; it.off = it.rb * 64;
        }
    } else {
        it.proj = ph == PH_O ? W_O : (ph == PH_GU ? W_GATE : W_DOWN);
        it.rb = it.group;
        it.off = it.group * 64;
    }
    // O runs while q and k are still being summed, so its rows and counters
    // lie past those of the QKV blocks (acc_base, cnt_base)
    it.arow = P.acc_base + it.group * 64;
    return it;
}

enum { DONE_QKV = 0, DONE_V = 1, DONE_O = 2, DONE_GU = 3, DONE_DOWN = 4, DONE_N = 5 };

// Wait until counter ctr reaches target.  Returns false when the wait gave
// up, or another workgroup's did (every wait is bounded).
__device__ bool wait_count(const ChainDev& C, const uint32_t* ctr, uint32_t target, int* flag_lds)
{
    __syncthreads();   // every thread has read the previous wait's flag
    if (threadIdx.x == 0) {
        uint32_t spins = 0;
        int ok = 1;
        for (;;) {
            // both loads in flight together: one memory round trip per poll
            const uint32_t c = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int e = __hip_atomic_load(C.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (c >= target) break;
            if (e) {
                ok = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(TQ_CHAIN_SLEEP);
            if (++spins >= kSpinLimit) {
                __hip_atomic_store(C.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ok = 0;
                break;
            }
        }
        *flag_lds = ok;
    }
    __syncthreads();
    return *flag_lds != 0;
}

__device__ __forceinline__ double wave_sum_f64(double v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// The element of the phase input that position i reads (global memory
// written by the previous phase): x, x1, act, or for O repeat(v) -- query
// head h reads KV head h / (n_heads / n_kv).  `src` is the phase's base.
__device__ __forceinline__ const float* phase_source(const ChainDev& C, int ph, const float* x)
{
    return ph == PH_QKV ? x : (ph == PH_GU ? C.x1 : (ph == PH_DOWN ? C.act : C.qkv + C.nq + C.nkv));
}

// RMSNorm of the phase input with weight w, then the per-token absmax int8
// quantisation, into LDS (xq, zero-padded to whole 64-column chunks) and
// *sx.  The steps are tq.h's; every workgroup computes the same bytes.  A
// thread holds its kPer inputs and weights in registers.  Every load is
// issued before the first use and none sits under a branch (positions past
// n read element n - 1 and are zeroed afterwards): behind branches each
// load waited for the one before, one memory round trip per element.
constexpr int kPer = kMaxWidth / kThreads;

// The O phase's element positions (repeat(v)) of this thread, computed once
// per launch: the integer divisions would otherwise recur in every layer.
__device__ __forceinline__ void o_positions(const ChainDev& C, int (&o_at)[kPer])
{
    const int group = C.n_heads / C.n_kv, n = C.nq;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int i = min((int)threadIdx.x + j * kThreads, n - 1);
        const int head = i / C.head_dim, d = i - head * C.head_dim;
        o_at[j] = (head / group) * C.head_dim + d;
    }
}

__device__ void norm_quant(const ChainDev& C, int ph, const float* x, const float* w, int n, int8_t* xq,
                           float* sx, double* red_d, float* red_f, const int (&o_at)[kPer])
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float* src = phase_source(C, ph, x);
    int at[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) at[j] = ph == PH_O ? o_at[j] : min(tid + j * kThreads, n - 1);
    float v[kPer], wt[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        v[j] = ld_shared(src + at[j]);
        wt[j] = w[min(tid + j * kThreads, n - 1)];
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const bool in = tid + j * kThreads < n;
        v[j] = in ? v[j] : 0.0f;
        wt[j] = in ? wt[j] : 0.0f;
    }
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) ss += (double)v[j] * (double)v[j];
    ss = wave_sum_f64(ss);
    if (lane == 0) red_d[wave] = ss;
    __syncthreads();
    ss = 0.0;
    for (int k = 0; k < kWaves; ++k) ss += red_d[k];
    const float ms = (float)(ss / (double)n);
    const float r = 1.0f / sqrtf(ms + C.eps);
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        v[j] = __fmul_rn(__fmul_rn(v[j], r), wt[j]);   // zero past n
        a = fmaxf(a, fabsf(v[j]));
    }
    a = wave_max(a);
    if (lane == 0) red_f[wave] = a;
    __syncthreads();
    a = red_f[0];
    for (int k = 1; k < kWaves; ++k) a = fmaxf(a, red_f[k]);
    const float inv = a > 0.0f ? 127.0f / a : 0.0f;
    const int npad = (n + TQ_CHUNK - 1) / TQ_CHUNK * TQ_CHUNK;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int i = tid + j * kThreads;
        if (i < npad) {
            float t = rintf(__fmul_rn(v[j], inv));
            t = fminf(fmaxf(t, -127.0f), 127.0f);
            xq[i] = (int8_t)(int)t;
        }
    }
    if (tid == 0) *sx = a > 0.0f ? a / 127.0f : 0.0f;
    __syncthreads();
}

#ifndef TQ_CHAIN_DEPTH
#define TQ_CHAIN_DEPTH 2     // chunks in flight per wave (measured: 4, 6 and 8 were no faster; the
                             // phase time is in the barrier, the input's round trip and the stores)
#endif
using RB = RowBlock<TQ_F32_Q8, TQ_SCALE_TENSOR, 1, 1, TQ_CHAIN_DEPTH>;

// The chunk range of this wave within an item: split s of the block's NC
// chunks, then this wave's share among `nw` waves.
__device__ __forceinline__ void wave_range(int NC, int splits, int s, int nw, int w, int* c0, int* c1)
{
    const int a = (int)((int64_t)NC * s / splits), b = (int)((int64_t)NC * (s + 1) / splits);
    *c0 = a + (int)((int64_t)(b - a) * w / nw);
    *c1 = a + (int)((int64_t)(b - a) * (w + 1) / nw);
}

__global__ __launch_bounds__(kThreads) void k_bitnet_chain(const ChainDev* __restrict__ Cp, float* x, float* qkv_out)
{
    const ChainDev C = ld_uniform_struct(Cp);
    __shared__ __attribute__((aligned(16))) int8_t xq[kMaxWidth];
    __shared__ int32_t red[kWaves][64];
    __shared__ double red_d[kWaves];
    __shared__ float red_f[kWaves];
    __shared__ float sx_lds;
    __shared__ int flag;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    int o_at[kPer];
    o_positions(C, o_at);

    for (int l = 0; l < C.n_layers; ++l) {
        const LayerDev& Ld = C.layers[l];
        for (int ph = 0; ph < 4; ++ph) {
            const PhaseDev P = ld_uniform_struct(&Cp->ph[ph]);
            // GU: waves 0..kWaves/2-1 run gate, the others up; else all waves one projection
            const int nw = ph == PH_GU ? kWaves / 2 : kWaves;
            const int wp = ph == PH_GU ? wave / nw : 0;
            const int ws = wave - wp * nw;
            const int first = blockIdx.x;
            if (first >= P.items) continue;      // no item in this phase
            Item it = item_of(C, P, ph, first);
            const tq_prob_dev& Pp = Ld.p[it.proj + wp];
            int c0 = 0, c1 = 0;
            wave_range(Pp.NC, P.splits, it.split, nw, ws, &c0, &c1);
            RB blk(Pp, it.rb, xq, nullptr);
            blk.begin(c0, c1);     // the codes stream in during the wait
            uint32_t* dl = C.done + l * DONE_N;
            bool ok = true;
            if (ph == PH_QKV) {
                if (l > 0) ok = wait_count(C, dl - DONE_N + DONE_DOWN, (uint32_t)C.ph[PH_DOWN].groups, &flag);
            } else if (ph == PH_O) {
                ok = wait_count(C, dl + DONE_V, (uint32_t)C.nb_kv, &flag);
            } else if (ph == PH_GU) {
                // x1 complete; and every QKV block, so that no workgroup still
                // reads x when DOWN rewrites it
                ok = wait_count(C, dl + DONE_O, (uint32_t)C.ph[PH_O].groups, &flag) &&
                     wait_count(C, dl + DONE_QKV, (uint32_t)C.ph[PH_QKV].groups, &flag);
            } else {
                ok = wait_count(C, dl + DONE_GU, (uint32_t)C.ph[PH_GU].groups, &flag);
            }
            if (!ok) return;
            norm_quant(C, ph, x, Ld.norm[ph], P.width, xq, &sx_lds, red_d, (float*)red_f, o_at);
            const float sx = sx_lds;
            for (int item = first; item < P.items; item += C.G) {
                int part;
                if (item == first) {
                    blk.finish(nullptr);
                    part = blk.p[0][0];
                } else {
                    it = item_of(C, P, ph, item);
                    const tq_prob_dev& Pq = Ld.p[it.proj + wp];
                    wave_range(Pq.NC, P.splits, it.split, nw, ws, &c0, &c1);
                    RB b2(Pq, it.rb, xq, nullptr);
                    b2.run(c0, c1, nullptr);
                    part = b2.p[0][0];
                }
                // the waves' partial sums, per projection, in wave order
                red[wave][lane] = part;
                __syncthreads();
                if (wave == 0) {
                    int sa = 0, sb = 0;
                    for (int k = 0; k < nw; ++k) sa += red[k][lane];
                    if (ph == PH_GU)
                        for (int k = nw; k < kWaves; ++k) sb += red[k][lane];
                    const int ra = it.arow + lane;                  // accumulator rows
                    const int rbw = ra + C.ph[PH_GU].groups * 64;   // GU: up's rows past gate's
                    bool last = true;
                    if (P.splits > 1) {
                        __hip_atomic_fetch_add(C.acc + ra, sa, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        if (ph == PH_GU) __hip_atomic_fetch_add(C.acc + rbw, sb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        wait_stores();     // the partial sums are in before the count says so
                        uint32_t old = 0;
                        if (lane == 0)
                            old = __hip_atomic_fetch_add(C.cnt + P.cnt_base + it.group, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        old = __shfl(old, 0, 64);
                        last = old == (uint32_t)P.splits - 1;
                        if (last) {
                            sa = __hip_atomic_exchange(C.acc + ra, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            if (ph == PH_GU) sb = __hip_atomic_exchange(C.acc + rbw, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            if (lane == 0) __hip_atomic_store(C.cnt + P.cnt_base + it.group, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        }
                    }
                    const tq_prob_dev& Pa = Ld.p[it.proj];
                    const int n = it.rb * 64 + lane;
                    if (last && n < Pa.N) {
                        const float ca = __fmul_rn(ld_uniform((const float*)Pa.scales), sx);
                        const float ya = __fmul_rn((float)sa, ca);
                        if (ph == PH_QKV) {
                            st_shared(C.qkv + it.off + lane, ya);
                            if (qkv_out) qkv_out[(int64_t)l * (C.nq + 2 * C.nkv) + it.off + lane] = ya;
                        } else if (ph == PH_O) {
                            st_shared(C.x1 + n, __fadd_rn(ld_shared(x + n), ya));
                        } else if (ph == PH_GU) {
                            const tq_prob_dev& Pb = Ld.p[W_UP];
                            const float cb = __fmul_rn(ld_uniform((const float*)Pb.scales), sx);
                            const float u = __fmul_rn((float)sb, cb);
                            const float g = fmaxf(ya, 0.0f);
                            st_shared(C.act + n, __fmul_rn(__fmul_rn(g, g), u));
                        } else {
                            st_shared(x + n, __fadd_rn(ld_shared(C.x1 + n), ya));
                        }
                    }
                    if (last) {   // the block is written: count it once its stores are complete
                        wait_stores();
                        if (lane == 0) {
                            const int c = ph == PH_QKV ? DONE_QKV : (ph == PH_O ? DONE_O : (ph == PH_GU ? DONE_GU : DONE_DOWN));
                            __hip_atomic_fetch_add(dl + c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            if (ph == PH_QKV && it.proj == W_V)
                                __hip_atomic_fetch_add(dl + DONE_V, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        }
                    }
                }
                __syncthreads();
            }
        }
    }
}

__global__ void k_chain_reset(ChainDev* C, int acc_n, int cnt_n)
{
    const ChainDev c = *C;
    for (int i = threadIdx.x; i < acc_n; i += blockDim.x) c.acc[i] = 0;
    for (int i = threadIdx.x; i < cnt_n; i += blockDim.x) c.cnt[i] = 0;
    for (int i = threadIdx.x; i < c.n_layers * DONE_N; i += blockDim.x) c.done[i] = 0;
    if (threadIdx.x == 0) *c.err = 0;
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
struct Sizes {
    int64_t nq, nkv, acc_n, cnt_n;
    int64_t off_layers, off_qkv, off_x1, off_act, off_acc, off_cnt, off_done, off_err, total;
};

tq_status check_dims(const tq_bitnet_dims* d, int32_t n_layers)
{
    if (!d) return tq_fail(TQ_ERR_ARG, "dims is NULL");
    if (n_layers < 1) return tq_fail(TQ_ERR_ARG, "n_layers = %d", n_layers);
    if (d->hidden < 16 || d->intermediate < 16 || d->n_heads < 1 || d->n_kv_heads < 1 || d->head_dim < 1)
        return tq_fail(TQ_ERR_SHAPE, "non-positive dimension");
    if (d->n_heads % d->n_kv_heads != 0)
        return tq_fail(TQ_ERR_SHAPE, "n_heads %d not a multiple of n_kv_heads %d", d->n_heads, d->n_kv_heads);
    if ((int64_t)d->n_heads * d->head_dim != d->hidden)
        return tq_fail(TQ_ERR_SHAPE, "n_heads * head_dim = %lld, hidden = %d",
                       (long long)d->n_heads * d->head_dim, d->hidden);
    if (d->hidden % 16 || d->intermediate % 16 || ((int64_t)d->n_kv_heads * d->head_dim) % 16)
        return tq_fail(TQ_ERR_SHAPE, "widths must be multiples of 16");
    if (d->hidden > kMaxWidth || d->intermediate > kMaxWidth)
        return tq_fail(TQ_ERR_UNSUPPORTED, "widths above %d", kMaxWidth);
    if (!(d->eps >= 0.0f) || !std::isfinite(d->eps)) return tq_fail(TQ_ERR_VALUE, "eps must be finite and >= 0");
    return TQ_OK;
}

Sizes sizes_of(const tq_bitnet_dims* d, int32_t n_layers)
{
    Sizes s;
    s.nq = (int64_t)d->n_heads * d->head_dim;
    s.nkv = (int64_t)d->n_kv_heads * d->head_dim;
    // blocks: QKV (q, k, v), then O's own range after them; GU (gate, then up);
    // DOWN -- 64 accumulator rows and one counter per block
    const int64_t nb_qkv = (s.nq + 63) / 64 + 2 * ((s.nkv + 63) / 64);
    const int64_t nb_h = ((int64_t)d->hidden + 63) / 64, nb_i = ((int64_t)d->intermediate + 63) / 64;
    s.acc_n = 64 * std::max({nb_qkv + nb_h, 2 * nb_i, nb_h});
    s.cnt_n = std::max({nb_qkv + nb_h, nb_i, nb_h});
    int64_t o = tq_align256(sizeof(ChainDev));
    s.off_layers = o;
    o = tq_align256(o + (int64_t)n_layers * sizeof(LayerDev));
    s.off_qkv = o;
    o = tq_align256(o + 4 * (s.nq + 2 * s.nkv));
    s.off_x1 = o;
    o = tq_align256(o + 4 * (int64_t)d->hidden);
    s.off_act = o;
    o = tq_align256(o + 4 * (int64_t)d->intermediate);
    s.off_acc = o;
    o = tq_align256(o + 4 * s.acc_n);
    s.off_cnt = o;
    o = tq_align256(o + 4 * s.cnt_n);
    s.off_done = o;
    o = tq_align256(o + 4 * (int64_t)n_layers * DONE_N);
    s.off_err = o;
    s.total = tq_align256(o + 4);
    return s;
}

int grid_limit()
{
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_bitnet_chain, kThreads, 0) != hipSuccess)
        return 0;
    return per_cu * tq_device_cus();
}

}  // namespace

TQ_EXPORT tq_status tq_bitnet_chain_workspace_size(const tq_bitnet_dims* dims, int32_t n_layers, size_t* bytes)
{
    if (!bytes) return tq_fail(TQ_ERR_ARG, "bytes is NULL");
    tq_status s = check_dims(dims, n_layers);
    if (s) return s;
    *bytes = (size_t)sizes_of(dims, n_layers).total;
    return tq_ok();
}

TQ_EXPORT tq_status tq_bitnet_chain_prepare(const tq_bitnet_dims* dims, const tq_bitnet_layer* layers,
                                            int32_t n_layers, void* workspace, size_t workspace_bytes,
                                            tq_chain_plan* plan, void* stream)
{
    if (!plan) return tq_fail(TQ_ERR_ARG, "plan is NULL");
    tq_status s = check_dims(dims, n_layers);
    if (s) return s;
    if (!layers) return tq_fail(TQ_ERR_ARG, "layers is NULL");
    if ((s = tq_check_ptr(workspace, "workspace", false, 256))) return s;
    const Sizes z = sizes_of(dims, n_layers);
    if ((int64_t)workspace_bytes < z.total)
        return tq_fail(TQ_ERR_ARG, "workspace has %zu bytes, needs %lld", workspace_bytes, (long long)z.total);
    hipStream_t st = (hipStream_t)stream;
    const int64_t hid = dims->hidden, inter = dims->intermediate;
    const int64_t shape[7][2] = {{z.nq, hid}, {z.nkv, hid}, {z.nkv, hid}, {hid, z.nq},
                                 {inter, hid}, {inter, hid}, {hid, inter}};
    static const char* names[7] = {"q", "k", "v", "o", "gate", "up", "down"};
    std::vector<LayerDev> ld((size_t)n_layers);
    std::vector<tq_blob_header> hdr((size_t)n_layers * 7);
    for (int32_t l = 0; l < n_layers; ++l) {
        for (int p = 0; p < 7; ++p) {
            if ((s = tq_check_ptr(layers[l].w[p], names[p], false))) return tq_fail(s, "layer %d: blob %s", l, names[p]);
            if ((s = tq_check_hip(hipMemcpyAsync(&hdr[(size_t)l * 7 + p], layers[l].w[p], sizeof(tq_blob_header),
                                                 hipMemcpyDeviceToHost, st), "tq_bitnet_chain_prepare header")))
                return s;
        }
        for (int j = 0; j < 4; ++j)
            if ((s = tq_check_ptr(layers[l].norm[j], "norm", false, 4))) return tq_fail(s, "layer %d: norm %d", l, j);
    }
    if ((s = tq_check_hip(hipStreamSynchronize(st), "tq_bitnet_chain_prepare synchronize"))) return s;
    for (int32_t l = 0; l < n_layers; ++l) {
        for (int p = 0; p < 7; ++p) {
            const tq_blob_header& h = hdr[(size_t)l * 7 + p];
            tq_weight_desc d;
            memset(&d, 0, sizeof d);
            d.planes = 1;
            d.group = 0;
            d.scale_layout = TQ_SCALE_TENSOR;
            d.out_features = shape[p][0];
            d.in_features = shape[p][1];
            if (h.magic != TQ_BLOB_MAGIC || h.planes != 1 || h.scale_layout != TQ_SCALE_TENSOR ||
                h.out_features != d.out_features || h.in_features != d.in_features)
                return tq_fail(TQ_ERR_SHAPE, "layer %d: blob %s is not a one-plane per-tensor %lld x %lld weight", l,
                               names[p], (long long)d.out_features, (long long)d.in_features);
            if (h.pack_status != 0) return tq_fail(TQ_ERR_VALUE, "layer %d: blob %s was not packed cleanly", l, names[p]);
            tq_layout L;
            if ((s = tq_check_desc(&d, &L))) return s;
            ld[(size_t)l].p[p] = tq_make_prob(L, layers[l].w[p], 1, nullptr, nullptr, nullptr, nullptr);
        }
        for (int j = 0; j < 4; ++j) ld[(size_t)l].norm[j] = layers[l].norm[j];
    }
    int G = plan->workgroups;
    const int lim = grid_limit();
    if (lim <= 0) return tq_fail(TQ_ERR_DEVICE, "no occupancy for the chain kernel");
    // default: one workgroup per two compute units -- enough items for every
    // phase of the BitNet shapes, and a cheaper barrier than one per unit
    // (measured 1.64 ms per token against 2.0 ms with 256)
    if (G <= 0) G = std::min(lim, std::max(1, tq_device_cus() / 2));
    if (G > lim) return tq_fail(TQ_ERR_UNSUPPORTED, "%d workgroups requested, %d fit at once", G, lim);

    uint8_t* ws = (uint8_t*)workspace;
    ChainDev c;
    memset(&c, 0, sizeof c);
    c.n_layers = n_layers;
    c.hidden = dims->hidden;
    c.inter = dims->intermediate;
    c.n_heads = dims->n_heads;
    c.n_kv = dims->n_kv_heads;
    c.head_dim = dims->head_dim;
    c.nq = (int32_t)z.nq;
    c.nkv = (int32_t)z.nkv;
    c.nb_q = (int32_t)((z.nq + 63) / 64);
    c.nb_kv = (int32_t)((z.nkv + 63) / 64);
    c.G = G;
    c.eps = dims->eps;
    // blocks and column splits per phase: enough items to give every
    // workgroup one, each wave keeping at least one 64-column chunk
    const int64_t groups[4] = {c.nb_q + 2 * c.nb_kv, (hid + 63) / 64, (inter + 63) / 64, (hid + 63) / 64};
    const int64_t chunks[4] = {(hid + 63) / 64, (z.nq + 63) / 64, (hid + 63) / 64, (inter + 63) / 64};
    const int64_t width[4] = {hid, z.nq, hid, inter};
    for (int ph = 0; ph < 4; ++ph) {
        const int nw = ph == PH_GU ? kWaves / 2 : kWaves;
        int64_t S = std::max<int64_t>(1, G / groups[ph]);
        S = std::min<int64_t>(S, std::max<int64_t>(1, chunks[ph] / nw));
        c.ph[ph].groups = (int32_t)groups[ph];
        c.ph[ph].splits = (int32_t)S;
        c.ph[ph].items = (int32_t)(groups[ph] * S);
        c.ph[ph].width = (int32_t)width[ph];
        c.ph[ph].acc_base = ph == PH_O ? (int32_t)(64 * groups[PH_QKV]) : 0;
        c.ph[ph].cnt_base = ph == PH_O ? (int32_t)groups[PH_QKV] : 0;
    }
    c.layers = (const LayerDev*)(ws + z.off_layers);
    c.qkv = (float*)(ws + z.off_qkv);
    c.x1 = (float*)(ws + z.off_x1);
    c.act = (float*)(ws + z.off_act);
    c.acc = (int32_t*)(ws + z.off_acc);
    c.cnt = (uint32_t*)(ws + z.off_cnt);
    c.done = (uint32_t*)(ws + z.off_done);
    c.err = (int32_t*)(ws + z.off_err);
    std::vector<uint8_t> host((size_t)z.off_qkv, 0);
    memcpy(host.data(), &c, sizeof c);
    memcpy(host.data() + z.off_layers, ld.data(), ld.size() * sizeof(LayerDev));
    if ((s = tq_check_hip(hipMemsetAsync(ws + z.off_qkv, 0, (size_t)(z.total - z.off_qkv), st), "tq_bitnet_chain_prepare clear")))
        return s;
    if ((s = tq_check_hip(hipMemcpyAsync(ws, host.data(), host.size(), hipMemcpyHostToDevice, st),
                          "tq_bitnet_chain_prepare copy")))
        return s;
    if ((s = tq_check_hip(hipStreamSynchronize(st), "tq_bitnet_chain_prepare synchronize"))) return s;
    memset(plan, 0, sizeof *plan);
    plan->workspace = workspace;
    plan->n_layers = n_layers;
    plan->workgroups = G;
    plan->dims = *dims;
    return tq_ok();
}

TQ_EXPORT tq_status tq_bitnet_chain_run(const tq_chain_plan* plan, float* x, float* qkv, void* stream)
{
    if (!plan || !plan->workspace || plan->n_layers < 1 || plan->workgroups < 1)
        return tq_fail(TQ_ERR_ARG, "plan is not filled by tq_bitnet_chain_prepare");
    tq_status s;
    if ((s = tq_check_ptr(x, "x", false, 4))) return s;
    if ((s = tq_check_ptr(qkv, "qkv", true, 4))) return s;
    const Sizes z = sizes_of(&plan->dims, plan->n_layers);
    hipStream_t st = (hipStream_t)stream;
    ChainDev* c = (ChainDev*)plan->workspace;
    hipLaunchKernelGGL(k_chain_reset, dim3(1), dim3(256), 0, st, c, (int)z.acc_n, (int)z.cnt_n);
    if ((s = tq_check_launch("tq_bitnet_chain_run reset"))) return s;
    const ChainDev* cp = c;
    void* args[] = {(void*)&cp, (void*)&x, (void*)&qkv};
    if ((s = tq_check_hip(hipLaunchCooperativeKernel((const void*)k_bitnet_chain, dim3(plan->workgroups),
                                                     dim3(kThreads), args, 0, st),
                          "tq_bitnet_chain_run launch")))
        return s;
    return tq_ok();
}

TQ_EXPORT tq_status tq_bitnet_chain_status(const tq_chain_plan* plan, void* stream)
{
    if (!plan || !plan->workspace) return tq_fail(TQ_ERR_ARG, "plan is not filled by tq_bitnet_chain_prepare");
    hipStream_t st = (hipStream_t)stream;
    const Sizes z = sizes_of(&plan->dims, plan->n_layers);
    int32_t err = 0;
    tq_status s;
    if ((s = tq_check_hip(hipMemcpyAsync(&err, (const uint8_t*)plan->workspace + z.off_err, 4,
                                         hipMemcpyDeviceToHost, st), "tq_bitnet_chain_status copy")))
        return s;
    if ((s = tq_check_hip(hipStreamSynchronize(st), "tq_bitnet_chain_status synchronize"))) return s;
    if (err) return tq_fail(TQ_ERR_DEVICE, "a chain wait gave up (the grid was not all resident)");
    return tq_ok();
}
