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
//      meet in LDS; the item stores its block's int32 partial sums to a slot
//      of its own (split, row) and counts the item done.
// Nobody adds the splits of a block or applies its epilogue at the end of a
// phase: the next phase's workgroups read every split's slot along with the
// rest of their input, add them (int32, exact in any order) and apply the
// epilogue themselves (fl(float(sum) * fl(s_w * s_x)), the residual add or
// relu2(gate) * up), the same operations in the same order, so the bits are
// those of a single writer.  A phase's critical path is then the slot
// stores and the count, the consumer's poll and one read of its input:
// three memory round trips, where a last-split reduction (atomic adds, an
// arrival count that returns, an exchange, the output stores) took six or
// seven.  The residual vectors that later phases need whole (x, x1) are
// stored by designated workgroups, and workgroup 0 publishes each phase's
// input scale s_x.
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
#define TQ_CHAIN_SLEEP 32                    // s_sleep between two polls of a wait (units of 64 cycles)
#endif

enum { PH_QKV = 0, PH_O = 1, PH_GU = 2, PH_DOWN = 3 };
enum { W_Q = 0, W_K, W_V, W_O, W_GATE, W_UP, W_DOWN };

struct LayerDev {
    tq_prob_dev p[7];
    const float* norm[4];
};

#ifndef TQ_CHAIN_SPLITS
#define TQ_CHAIN_SPLITS 3
#endif
#ifndef TQ_CHAIN_SPLITS_GU
#define TQ_CHAIN_SPLITS_GU 2
#endif
constexpr int kMaxSplits = TQ_CHAIN_SPLITS;      // column splits of a block (the consumers add this many slots at most)
constexpr int kMaxSplitsGU = TQ_CHAIN_SPLITS_GU; // GU's: DOWN's input reads two slot vectors (gate, up), so half as many

struct PhaseDev {
    int32_t groups;     // output blocks: 64-row blocks (QKV over q|k|v; GU: gate/up pairs)
    int32_t splits;     // column splits per block, 1 .. kMaxSplits
    int32_t items;      // groups * splits
    int32_t width;      // input length
    int32_t prow;       // rows of one split's partial sums (QKV: q|k|v; GU: gate|up)
    int32_t pbase;      // the phase's first slot: split s, row r at part[pbase + s prow + r]
};

struct ChainDev {
    PhaseDev ph[4];
    int32_t n_layers, hidden, inter, n_heads, n_kv, head_dim;
    int32_t nq, nkv, nb_q, nb_kv, G;
    float eps;
    const LayerDev* layers;
    float* x1;          // [hidden] x + o of the current layer (the residual of DOWN)
    int32_t* part;      // the phases' int32 partial sums per split and row
    float* sxs;         // [n_layers][4] the int8 scale of each phase's input
    uint32_t* done;     // [n_layers][5] items written: QKV, v, O, GU, DOWN
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
__device__ __forceinline__ int32_t ld_shared_i32(const int32_t* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_shared_i32(int32_t* p, int32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The same accesses through a buffer resource: the byte offset within the
// buffer is one 32-bit VGPR where a global access takes a 64-bit address in
// two, and a uniform offset rides in an SGPR.  The phase inputs keep dozens
// of loads in flight per thread, so this halves their address registers.
// Cache policy sc1 is the agent scope of the accesses above.  They are
// ordered after a wait by the barrier that ends it, as any memory access.
constexpr int kAgent = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* p)
{
    // every buffer here is far below 4 GiB; dword 3 is gfx9's raw-dword format
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, -1, 0x00020000);
}
__device__ __forceinline__ int32_t ld_buf_i32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, kAgent);
}
__device__ __forceinline__ float ld_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __int_as_float(ld_buf_i32(r, voff, soff));
}
__device__ __forceinline__ void st_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, float v)
{
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(v), r, (int)voff, 0, kAgent);
}
// Wait until this wave's stores and atomics have completed.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

struct Item {
    int proj;           // projection of waves 0 .. kWaves/2 - 1 (GU) or of all waves
    int rb;             // 64-row block within the projection
    int split;
    int group;
    int off;            // first output row of the block (in q|k|v for QKV; of gate for GU)
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
    return it;
}

enum { DONE_QKV = 0, DONE_V = 1, DONE_O = 2, DONE_GU = 3, DONE_DOWN = 4, DONE_N = 5 };
#ifndef TQ_CHAIN_CTR_STRIDE
#define TQ_CHAIN_CTR_STRIDE 64
#endif
// Counter c of layer l, each in a 256-byte line of its own: the polls of one
// counter then do not queue behind the increments of another.
constexpr int kCtrStride = TQ_CHAIN_CTR_STRIDE;   // dwords
#ifndef TQ_CHAIN_ERR_EVERY
#define TQ_CHAIN_ERR_EVERY 16
#endif
constexpr uint32_t kErrEvery = TQ_CHAIN_ERR_EVERY;   // a power of two
__device__ __forceinline__ uint32_t* counter(const ChainDev& C, int l, int c)
{
    return C.done + (l * DONE_N + c) * kCtrStride;
}

// Wait until counter ctr reaches target.  Returns false when the wait gave
// up, or another workgroup's did (every wait is bounded).
// A counter poll: a relaxed agent-scope load through the global address
// space (a flat load also waits on the LDS counter).
__device__ __forceinline__ uint32_t poll(const uint32_t* p)
{
    return __hip_atomic_load((const __attribute__((address_space(1))) uint32_t*)p, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

__device__ bool wait_count(const ChainDev& C, const uint32_t* ctr, uint32_t target, int* flag_lds)
{
    __syncthreads();   // every thread has read the previous wait's flag
    if (threadIdx.x == 0) {
        uint32_t spins = 0;
        int ok = 1;
        for (;;) {
            if (poll(ctr) >= target) break;
            // the error flag, which every waiting workgroup would otherwise
            // poll on one line, only every kErrEvery polls
            if ((spins & (kErrEvery - 1)) == kErrEvery - 1 && poll((const uint32_t*)C.err)) {
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

// Wave reductions with DPP moves inside each 16-lane row (pairs, quads,
// halves, rows) and four lane reads across the rows: no LDS round trip,
// where a shuffle per step (ds_bpermute) costs one in a dependent chain.
// Every lane returns the same value, in a fixed order of operations.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v)
{
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint64_t lo = dpp<CTRL>((uint32_t)u), hi = dpp<CTRL>((uint32_t)(u >> 32));
    return __longlong_as_double((long long)(lo | (hi << 32)));
}
__device__ __forceinline__ double readlane_f64(double v, int l)
{
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __longlong_as_double((long long)(lo | (hi << 32)));
}
enum { kDppSwap1 = 0xB1, kDppSwap2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140 };
__device__ __forceinline__ double wave_sum_f64(double v)
{
    v += dpp_f64<kDppSwap1>(v);        // quad_perm [1,0,3,2]
    v += dpp_f64<kDppSwap2>(v);        // quad_perm [2,3,0,1]: the quad's sum
    v += dpp_f64<kDppHalfMirror>(v);   // lane i <- 7 - i: the 8 lanes' sum
    v += dpp_f64<kDppMirror>(v);       // lane i <- 15 - i: the row's sum
    return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}
__device__ __forceinline__ float wave_max_dpp(float v)
{
    v = fmaxf(v, __uint_as_float(dpp<kDppSwap1>(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp<kDppSwap2>(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp<kDppHalfMirror>(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp<kDppMirror>(__float_as_uint(v))));
    const float a = fmaxf(__uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 0)),
                          __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 16)));
    const float b = fmaxf(__uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 32)),
                          __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 48)));
    return fmaxf(a, b);
}

// RMSNorm of the phase input with weight w, then the per-token absmax int8
// quantisation, into LDS (xq, zero-padded to whole 64-column chunks) and
// *sx.  The steps are tq.h's; every workgroup computes the same bytes.  A
// thread holds 4 R inputs and weights in registers, as R runs of four
// consecutive elements (from 4 (tid + j kThreads)), each read with one
// 16-byte load: a vector is R loads per thread (R = 2 up to 4096 wide, else
// 4), and a phase's loads stay within the 63 a wave can have outstanding.  Every load is issued before
// the first use and none sits under a branch (runs past n read the last
// run and are zeroed afterwards): behind branches each load waited for the
// one before.
constexpr int kPer = kMaxWidth / kThreads;
constexpr int kRuns = kPer / 4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int AUX = kAgent>
__device__ __forceinline__ u32x4 ld_buf4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, AUX);
}
__device__ __forceinline__ int run_start(int j, int n)
{
    return min(4 * ((int)threadIdx.x + j * kThreads), n - 4);
}

// The O phase's input runs (repeat(v)) of this thread as byte offsets into
// v, computed once per launch: the integer divisions would otherwise recur
// in every layer.  A run stays within one head (head_dim is a multiple of 4).
__device__ __forceinline__ void o_positions(const ChainDev& C, uint32_t (&o_at)[kRuns])
{
    const int group = C.n_heads / C.n_kv;
#pragma unroll
    for (int j = 0; j < kRuns; ++j) {
        const int i = run_start(j, C.nq);
        const int head = i / C.head_dim, d = i - head * C.head_dim;
        o_at[j] = 4u * (uint32_t)((head / group) * C.head_dim + d);
    }
}

// The sum of a phase's S split slots at the runs of byte offsets off[j]
// (slot s at sbase + s sstep bytes): every load is issued before the first
// add (S fixed at compile time).
template <int S, int R>
__device__ __forceinline__ void slot_sums(__amdgpu_buffer_rsrc_t r, uint32_t sbase, uint32_t sstep,
                                          const uint32_t (&off)[kRuns], int32_t (&sum)[kPer])
{
    u32x4 t[S][kRuns];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int j = 0; j < R; ++j) t[s][j] = ld_buf4(r, off[j], sbase + s * sstep);
#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t a = t[0][j][k];
#pragma unroll
            for (int s = 1; s < S; ++s) a += t[s][j][k];
            sum[4 * j + k] = (int32_t)a;
        }
}
template <int MAXS, int R>
__device__ __forceinline__ void slot_sum(const ChainDev& C, int ph, int row0, const uint32_t (&off)[kRuns],
                                         int32_t (&sum)[kPer])
{
    const PhaseDev& P = C.ph[ph];
    const __amdgpu_buffer_rsrc_t r = rsrc_of(C.part);
    const uint32_t sbase = 4u * (uint32_t)(P.pbase + row0), sstep = 4u * (uint32_t)P.prow;
    if (P.splits == 1 || MAXS == 1) slot_sums<1, R>(r, sbase, sstep, off, sum);
    else if (P.splits == 2 || MAXS == 2) slot_sums<2, R>(r, sbase, sstep, off, sum);
    else if (P.splits == 3 || MAXS == 3) slot_sums<3, R>(r, sbase, sstep, off, sum);
    else slot_sums<MAXS, R>(r, sbase, sstep, off, sum);
}
// A vector's runs at byte offsets off[j], agent scope.
template <int R>
__device__ __forceinline__ void load_runs(const float* p, const uint32_t (&off)[kRuns], float (&v)[kPer])
{
    const __amdgpu_buffer_rsrc_t r = rsrc_of(p);
    u32x4 t[kRuns];
#pragma unroll
    for (int j = 0; j < R; ++j) t[j] = ld_buf4(r, off[j], 0);
#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k) v[4 * j + k] = __uint_as_float(t[j][k]);
}
// fl(s_w * s_x): the epilogue factor of a product of phase ph in layer l
// (the weight's per-tensor scale times the phase input's int8 scale, which
// workgroup 0 published)
__device__ __forceinline__ float epi_scale(const ChainDev& C, const LayerDev& L, int proj, int l, int ph)
{
    return __fmul_rn(ld_uniform((const float*)L.p[proj].scales), ld_shared(C.sxs + l * 4 + ph));
}

// The elements of this thread's runs (byte offsets off[j]) of phase ph's
// input in layer l, from what the earlier phases left in memory:
//   QKV   x (layer 0: the input; then x1 + down of the layer before)
//   O     repeat(v): v from the QKV slots
//   GU    x1 = x + o
//   DOWN  relu2(gate) * up
// each product fl(float(sum of the splits) * fl(s_w * s_x)).
template <int R>
__device__ __forceinline__ void phase_input(const ChainDev& C, int l, int ph, const float* x,
                                            const uint32_t (&off)[kRuns], float (&v)[kPer])
{
    int32_t a[kPer];
    if (ph == PH_QKV && l == 0) {
        load_runs<R>(x, off, v);
    } else if (ph == PH_QKV) {
        float r[kPer];
        load_runs<R>(C.x1, off, r);
        slot_sum<kMaxSplits, R>(C, PH_DOWN, 0, off, a);
        const float ca = epi_scale(C, C.layers[l - 1], W_DOWN, l - 1, PH_DOWN);
#pragma unroll
        for (int j = 0; j < 4 * R; ++j) v[j] = __fadd_rn(r[j], __fmul_rn((float)a[j], ca));
    } else if (ph == PH_O) {
        slot_sum<kMaxSplits, R>(C, PH_QKV, C.nq + C.nkv, off, a);
        const float ca = epi_scale(C, C.layers[l], W_V, l, PH_QKV);
#pragma unroll
        for (int j = 0; j < 4 * R; ++j) v[j] = __fmul_rn((float)a[j], ca);
    } else if (ph == PH_GU) {
        float r[kPer];
        load_runs<R>(x, off, r);
        slot_sum<kMaxSplits, R>(C, PH_O, 0, off, a);
        const float ca = epi_scale(C, C.layers[l], W_O, l, PH_O);
#pragma unroll
        for (int j = 0; j < 4 * R; ++j) v[j] = __fadd_rn(r[j], __fmul_rn((float)a[j], ca));
    } else {
        int32_t b[kPer];
        slot_sum<kMaxSplitsGU, R>(C, PH_GU, 0, off, a);
        slot_sum<kMaxSplitsGU, R>(C, PH_GU, C.inter, off, b);
        const float cg = epi_scale(C, C.layers[l], W_GATE, l, PH_GU);
        const float cu = epi_scale(C, C.layers[l], W_UP, l, PH_GU);
#pragma unroll
        for (int j = 0; j < 4 * R; ++j) {
            const float g = fmaxf(__fmul_rn((float)a[j], cg), 0.0f);
            const float u = __fmul_rn((float)b[j], cu);
            v[j] = __fmul_rn(__fmul_rn(g, g), u);
        }
    }
}

// The phase input (phase_input), then its RMSNorm with weight w and the
// per-token absmax int8 quantisation, into LDS (xq, zero-padded to whole
// 64-column chunks) and *sx.  The steps are tq.h's; every workgroup computes
// the same bytes.  On the way the workgroup stores the rows of the residual
// vectors it is designated for (QKV: x; GU: x1; block b by the workgroup
// b mod npart, npart the phase's participants) and workgroup 0 publishes
// s_x; each wave waits for these stores before the item is counted.
template <int R>
__device__ void norm_quant(const ChainDev& C, int l, int ph, float* x, const float* w, int n, int npart, int8_t* xq,
                           float* sx, double* red_d, float* red_f, const uint32_t (&o_at)[kRuns])
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t off[kRuns];
#pragma unroll
    for (int j = 0; j < R; ++j) off[j] = ph == PH_O ? o_at[j] : 4u * (uint32_t)run_start(j, n);
    float v[kPer], wt[kPer];
    {
        const __amdgpu_buffer_rsrc_t rw = rsrc_of(w);
        u32x4 t[kRuns];
#pragma unroll
        for (int j = 0; j < R; ++j) t[j] = ld_buf4<0>(rw, 4u * (uint32_t)run_start(j, n), 0);
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
            for (int k = 0; k < 4; ++k) wt[4 * j + k] = __uint_as_float(t[j][k]);
    }
    phase_input<R>(C, l, ph, x, off, v);
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const bool in = 4 * (tid + j * kThreads) < n;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[4 * j + k] = in ? v[4 * j + k] : 0.0f;
            wt[4 * j + k] = in ? wt[4 * j + k] : 0.0f;
        }
    }
    if ((ph == PH_QKV && l > 0) || ph == PH_GU) {
        const __amdgpu_buffer_rsrc_t rd = rsrc_of(ph == PH_QKV ? x : C.x1);
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int e = 4 * (tid + j * kThreads);
            if (e < n && (e >> 6) % npart == (int)blockIdx.x) {
                u32x4 q;
#pragma unroll
                for (int k = 0; k < 4; ++k) q[k] = __float_as_uint(v[4 * j + k]);
                __builtin_amdgcn_raw_buffer_store_b128(q, rd, (int)(4u * (uint32_t)e), 0, kAgent);
            }
        }
    }
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < 4 * R; ++j) ss += (double)v[j] * (double)v[j];
    ss = wave_sum_f64(ss);
    if (lane == 0) red_d[wave] = ss;
    __syncthreads();
    ss = 0.0;
    for (int k = 0; k < kWaves; ++k) ss += red_d[k];
    const float ms = (float)(ss / (double)n);
    const float r = 1.0f / sqrtf(ms + C.eps);
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 4 * R; ++j) {
        v[j] = __fmul_rn(__fmul_rn(v[j], r), wt[j]);   // zero past n
        a = fmaxf(a, fabsf(v[j]));
    }
    a = wave_max_dpp(a);
    if (lane == 0) red_f[wave] = a;
    __syncthreads();
    a = red_f[0];
    for (int k = 1; k < kWaves; ++k) a = fmaxf(a, red_f[k]);
    const float inv = a > 0.0f ? 127.0f / a : 0.0f;
    const int npad = (n + TQ_CHUNK - 1) / TQ_CHUNK * TQ_CHUNK;
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int e = 4 * (tid + j * kThreads);
        if (e < npad) {   // npad is a multiple of 4: a run is wholly in or out
            uint32_t q = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float t = rintf(__fmul_rn(v[4 * j + k], inv));
                t = fminf(fmaxf(t, -127.0f), 127.0f);
                q |= ((uint32_t)(int)t & 0xffu) << (8 * k);
            }
            *(uint32_t*)(xq + e) = q;
        }
    }
    const float sxv = a > 0.0f ? a / 127.0f : 0.0f;
    if (tid == 0) {
        *sx = sxv;
        if (blockIdx.x == 0) st_shared(C.sxs + l * 4 + ph, sxv);
    }
    __syncthreads();
}

#ifndef TQ_CHAIN_DEPTH
#define TQ_CHAIN_DEPTH 6     // chunks in flight per wave (measured: 2, 4, 6 and 8 within 1.3%; 6 best)
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

// The layer's q | k | v for the caller, from the QKV slots: wave w of the
// workgroup takes the 64-row blocks blockIdx + npart (w + kWaves i).  The
// designated workgroups (npart: those with both a GU and a DOWN item) call
// it in the DOWN phase before its wait, while they would idle: they waited
// for every QKV item in the GU phase, and the next layer's QKV items, which
// rewrite the slots, wait for their DOWN items.
__device__ void qkv_rows(const ChainDev& C, const LayerDev& Ld, int l, float* qkv_out)
{
    const int npart = min(min(C.ph[PH_GU].items, C.ph[PH_DOWN].items), C.G);
    if ((int)blockIdx.x >= npart) return;
    const int R = C.nq + 2 * C.nkv, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const float cq = epi_scale(C, Ld, W_Q, l, PH_QKV), ck = epi_scale(C, Ld, W_K, l, PH_QKV),
                cv = epi_scale(C, Ld, W_V, l, PH_QKV);
    const PhaseDev& Q = C.ph[PH_QKV];
    for (int blk = blockIdx.x + npart * wave; blk * 64 < R; blk += npart * kWaves) {
        const int i = blk * 64 + lane;
        if (i >= R) break;
        int32_t t[kMaxSplits];
#pragma unroll
        for (int sp = 0; sp < kMaxSplits; ++sp)
            t[sp] = sp < Q.splits ? ld_shared_i32(C.part + Q.pbase + sp * Q.prow + i) : 0;
        int32_t sum = 0;
#pragma unroll
        for (int sp = 0; sp < kMaxSplits; ++sp) sum += t[sp];
        const float ca = i < C.nq ? cq : (i < C.nq + C.nkv ? ck : cv);
        qkv_out[(int64_t)l * R + i] = __fmul_rn((float)sum, ca);
    }
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
    uint32_t o_at[kRuns];
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
            // the projection's descriptor in SGPRs: a descriptor loaded
            // into VGPRs makes every code load a waterfall loop that waits
            // for all loads in flight (one round trip per chunk)
            const tq_prob_dev Pp = ld_uniform_struct(&Ld.p[it.proj + wp]);
            int c0 = 0, c1 = 0;
            wave_range(Pp.NC, P.splits, it.split, nw, ws, &c0, &c1);
            int n_out = (int)ld_uniform_u32(&Ld.p[it.proj], offsetof(tq_prob_dev, N) / 4);   // output rows
            RB blk(Pp, it.rb, xq, nullptr);
            blk.begin(c0, c1);     // the codes stream in during the wait
            bool ok = true;
            if (ph == PH_QKV) {
                if (l > 0) ok = wait_count(C, counter(C, l - 1, DONE_DOWN), (uint32_t)C.ph[PH_DOWN].items, &flag);
            } else if (ph == PH_O) {
                ok = wait_count(C, counter(C, l, DONE_V), (uint32_t)(C.nb_kv * C.ph[PH_QKV].splits), &flag);
            } else if (ph == PH_GU) {
                // x1 = x + o needs every O item, and x the rows the QKV
                // workgroups store
                ok = wait_count(C, counter(C, l, DONE_O), (uint32_t)C.ph[PH_O].items, &flag) &&
                     wait_count(C, counter(C, l, DONE_QKV), (uint32_t)C.ph[PH_QKV].items, &flag);
            } else {
                if (qkv_out) qkv_rows(C, Ld, l, qkv_out);
                ok = wait_count(C, counter(C, l, DONE_GU), (uint32_t)C.ph[PH_GU].items, &flag);
            }
            if (!ok) return;
            // two runs per thread for widths up to 4096 (no work on padding)
            if (P.width <= 2 * 4 * kThreads)
                norm_quant<2>(C, l, ph, x, Ld.norm[ph], P.width, min(P.items, C.G), xq, &sx_lds, red_d, (float*)red_f, o_at);
            else
                norm_quant<kRuns>(C, l, ph, x, Ld.norm[ph], P.width, min(P.items, C.G), xq, &sx_lds, red_d, (float*)red_f, o_at);
            for (int item = first; item < P.items; item += C.G) {
                int part;
                if (item == first) {
                    blk.finish(nullptr);
                    part = blk.p[0][0];
                } else {
                    it = item_of(C, P, ph, item);
                    const tq_prob_dev Pq = ld_uniform_struct(&Ld.p[it.proj + wp]);
                    wave_range(Pq.NC, P.splits, it.split, nw, ws, &c0, &c1);
                    n_out = (int)ld_uniform_u32(&Ld.p[it.proj], offsetof(tq_prob_dev, N) / 4);
                    RB b2(Pq, it.rb, xq, nullptr);
                    b2.run(c0, c1, nullptr);
                    part = b2.p[0][0];
                }
                // the waves' partial sums, per projection, in wave order
                red[wave][lane] = part;
                // this wave's stores of norm_quant (designated rows, s_x)
                // complete behind the product; they are out before any item
                // of the workgroup is counted
                wait_stores();
                __syncthreads();
                if (wave == 0) {
                    int sa = 0, sb = 0;
                    for (int k = 0; k < nw; ++k) sa += red[k][lane];
                    if (ph == PH_GU)
                        for (int k = nw; k < kWaves; ++k) sb += red[k][lane];
                    // the item's slot: its split's partial sums of the block's rows
                    int32_t* slot = C.part + P.pbase + it.split * P.prow + it.off;
                    if (it.rb * 64 + lane < n_out) {
                        st_shared_i32(slot + lane, sa);
                        if (ph == PH_GU) st_shared_i32(slot + C.inter + lane, sb);
                    }
                    wait_stores();   // the slot is written before the count says so
                    if (lane == 0) {
                        const int c = ph == PH_QKV ? DONE_QKV : (ph == PH_O ? DONE_O : (ph == PH_GU ? DONE_GU : DONE_DOWN));
                        __hip_atomic_fetch_add(counter(C, l, c), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        if (ph == PH_QKV && it.proj == W_V)
                            __hip_atomic_fetch_add(counter(C, l, DONE_V), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
                __syncthreads();
            }
        }
    }
    // the hidden state after the last layer, x = x1 + down: wave w of every
    // workgroup takes the 64-row blocks b with b = blockIdx + G (w + kWaves i)
    const int L = C.n_layers - 1;
    if (!wait_count(C, counter(C, L, DONE_DOWN), (uint32_t)C.ph[PH_DOWN].items, &flag)) return;
    const float cd = epi_scale(C, C.layers[L], W_DOWN, L, PH_DOWN);
    const PhaseDev& D = C.ph[PH_DOWN];
    for (int blk = blockIdx.x + C.G * wave; blk * 64 < C.hidden; blk += C.G * kWaves) {
        const int i = blk * 64 + lane;
        if (i >= C.hidden) break;
        int32_t t[kMaxSplits];
#pragma unroll
        for (int sp = 0; sp < kMaxSplits; ++sp)
            t[sp] = sp < D.splits ? ld_shared_i32(C.part + D.pbase + sp * D.prow + i) : 0;
        int32_t sum = 0;
#pragma unroll
        for (int sp = 0; sp < kMaxSplits; ++sp) sum += t[sp];
        st_shared(x + i, __fadd_rn(ld_shared(C.x1 + i), __fmul_rn((float)sum, cd)));
    }
}

__global__ void k_chain_reset(ChainDev* C)
{
    const ChainDev c = *C;
    for (int i = threadIdx.x; i < c.n_layers * DONE_N; i += blockDim.x) c.done[i * kCtrStride] = 0;
    if (threadIdx.x == 0) *c.err = 0;
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
struct Sizes {
    int64_t nq, nkv;
    int64_t prow[4], pbase[4], part_n;   // each phase's slot rows and first slot; every slot
    int64_t off_layers, off_x1, off_part, off_sxs, off_done, off_err, total;
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
    if (d->head_dim % 4) return tq_fail(TQ_ERR_SHAPE, "head_dim %d not a multiple of 4", d->head_dim);
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
    // the slots of every phase, kMaxSplits per row: QKV (q|k|v), O, GU
    // (gate|up), DOWN, one after the other (no two phases share a slot)
    const int64_t prow[4] = {s.nq + 2 * s.nkv, d->hidden, 2 * (int64_t)d->intermediate, d->hidden};
    s.part_n = 0;
    for (int ph = 0; ph < 4; ++ph) {
        s.prow[ph] = prow[ph];
        s.pbase[ph] = s.part_n;
        s.part_n += kMaxSplits * prow[ph];
    }
    int64_t o = tq_align256(sizeof(ChainDev));
    s.off_layers = o;
    o = tq_align256(o + (int64_t)n_layers * sizeof(LayerDev));
    s.off_x1 = o;
    o = tq_align256(o + 4 * (int64_t)d->hidden);
    s.off_part = o;
    o = tq_align256(o + 4 * s.part_n);
    s.off_sxs = o;
    o = tq_align256(o + 4 * 4 * (int64_t)n_layers);
    s.off_done = o;
    o = tq_align256(o + 4 * (int64_t)n_layers * DONE_N * kCtrStride);
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
        S = std::min<int64_t>(S, ph == PH_GU ? kMaxSplitsGU : kMaxSplits);
        c.ph[ph].groups = (int32_t)groups[ph];
        c.ph[ph].splits = (int32_t)S;
        c.ph[ph].items = (int32_t)(groups[ph] * S);
        c.ph[ph].width = (int32_t)width[ph];
        c.ph[ph].prow = (int32_t)z.prow[ph];
        c.ph[ph].pbase = (int32_t)z.pbase[ph];
    }
    c.layers = (const LayerDev*)(ws + z.off_layers);
    c.x1 = (float*)(ws + z.off_x1);
    c.part = (int32_t*)(ws + z.off_part);
    c.sxs = (float*)(ws + z.off_sxs);
    c.done = (uint32_t*)(ws + z.off_done);
    c.err = (int32_t*)(ws + z.off_err);
    std::vector<uint8_t> host((size_t)z.off_x1, 0);
    memcpy(host.data(), &c, sizeof c);
    memcpy(host.data() + z.off_layers, ld.data(), ld.size() * sizeof(LayerDev));
    if ((s = tq_check_hip(hipMemsetAsync(ws + z.off_x1, 0, (size_t)(z.total - z.off_x1), st), "tq_bitnet_chain_prepare clear")))
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
    hipStream_t st = (hipStream_t)stream;
    ChainDev* c = (ChainDev*)plan->workspace;
    hipLaunchKernelGGL(k_chain_reset, dim3(1), dim3(256), 0, st, c);
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
