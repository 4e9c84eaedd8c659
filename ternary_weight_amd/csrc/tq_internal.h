// Host-side helpers shared by the libtq translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_layout.h"

#define TQ_EXPORT extern "C" __attribute__((visibility("default")))

// Record a message for tq_last_error() on this thread and return `s`.
tq_status tq_fail(tq_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the thread's last error; returns TQ_OK.
tq_status tq_ok();

// Validate a weight descriptor and fill the layout.
tq_status tq_check_desc(const tq_weight_desc* d, tq_layout* L);
// Device pointer checks: non-null unless `nullable`, aligned to `align` bytes.
tq_status tq_check_ptr(const void* p, const char* name, bool nullable, int align = 16);
// After a launch: map hipGetLastError() to TQ_ERR_DEVICE.
tq_status tq_check_launch(const char* what);
tq_status tq_check_hip(hipError_t e, const char* what);

// The device's compute-unit count (cached per device).
int tq_device_cus();

// Problem descriptor as the decode kernels read it (host fills, device reads).
struct tq_prob_dev {
    const uint8_t* codes;      // blob + codes_off
    const uint8_t* scales;     // blob + scales_off (indices for CODEBOOK)
    const uint16_t* cb;        // blob + cb_off (CODEBOOK) or null
    const void* x;             // [M][Kin]
    const float* x_scale;      // [M] (I8) or null
    float* y;                  // [M][N]
    int32_t* acc;              // optional [M][N]
    int32_t N, Kin;
    int32_t NC, NGD;
    int32_t NID, g;
    int32_t M, log2g;
};

// Call validation shared by the entry points (tq_entry.hip): x_type, M in
// 0..max_m, pointers (x aligned to x_align bytes), the acc restriction.
tq_status tq_check_call(const tq_layout& L, const void* blob, int64_t M, int32_t x_type, const void* x,
                        const float* x_scale, const float* y, const int32_t* acc, int64_t max_m,
                        int x_align = 4);
// The device-side descriptor of one problem.
tq_prob_dev tq_make_prob(const tq_layout& L, const void* blob, int64_t M, const void* x,
                         const float* x_scale, float* y, int32_t* acc);
// Prefix the thread's last error message with a problem index.
tq_status tq_fail_problem(tq_status s, int32_t i);

// bf16 decode with at least this many tokens runs on the matrix cores (the
// few-token kernels) when x is 16-byte aligned: 3, also for the codec's
// two-bit digit planes, whose matrix-core kernel combines the three digits
// into one operand (Llama-8B-shaped codec stack: 3 tokens 1.52 ms there
// against 1.63 ms on the vector ALUs, 2 tokens 1.5 against 1.31 ms), and 5
// for the compact codes, whose matrix-core kernel applies a scale after
// every 16 columns (4 tokens 0.98 ms on the vector ALUs, 5 tokens 1.83 ms
// there against 1.5 ms on the matrix cores).
#ifndef TQ_BF16_MFMA_MIN_M
#define TQ_BF16_MFMA_MIN_M 3
#endif
#ifndef TQ_BF16_MFMA_MIN_M_CODEC
#define TQ_BF16_MFMA_MIN_M_CODEC 3
#endif
#ifndef TQ_BF16_MFMA_MIN_M_B3
#define TQ_BF16_MFMA_MIN_M_B3 5
#endif
// int8 decode with at least this many tokens runs on the matrix cores (one
// pass over the codes for up to 16 tokens, where the vector ALUs take them
// 4 at a time), when the groups are whole 64-column steps and x is 16-byte
// aligned.
#ifndef TQ_I8_MFMA_MIN_M
#define TQ_I8_MFMA_MIN_M 2
#endif
static inline int64_t tq_bf16_mfma_min_m(int layout)
{
    return layout == TQ_SCALE_CODEBOOK ? TQ_BF16_MFMA_MIN_M_CODEC
                                       : (layout == TQ_SCALE_CODEBOOK_B3 ? TQ_BF16_MFMA_MIN_M_B3 : TQ_BF16_MFMA_MIN_M);
}
// The fewest tokens of a decode call that go to the matrix cores (x_type
// TQ_BF16 or TQ_I8; never for the others).
static inline int64_t tq_mfma_min_m(int x_type, int layout)
{
    return x_type == TQ_BF16 ? tq_bf16_mfma_min_m(layout) : (x_type == TQ_I8 ? TQ_I8_MFMA_MIN_M : INT64_MAX);
}
static inline bool tq_gemv_uses_mfma(int x_type, int layout, int64_t M, const void* x)
{
    return M >= tq_mfma_min_m(x_type, layout) && ((uintptr_t)x & 15) == 0;
}
// tq_gemm_grouped_prepare with per-problem token counts (tokens may be NULL:
// every problem has M); tq_gemm.hip.
tq_status tq_gemm_grouped_prepare_counts(const tq_problem* problems, const int32_t* tokens, int32_t count,
                                         int64_t M, int32_t x_type, void* workspace, size_t workspace_bytes,
                                         tq_grouped_plan* plan, void* stream);
// Matrix-core launch of one problem (tq_gemm.hip); the arguments are checked.
tq_status tq_gemm_launch(const tq_layout& L, const tq_prob_dev& P, int x_type, hipStream_t stream);
// Whether a matrix-core kernel takes this shape (every operand below the
// 4 GiB its 32-bit offsets reach); the decode entry points send a bf16 call
// that it does not take to the vector-ALU kernels instead.
bool tq_gemm_supports(const tq_layout& L, int x_type, int64_t M);

// Decode launch shared by tq_gemv and tq_gemv_grouped_run (tq_gemv.hip).
tq_status tq_gemv_launch_single(const tq_layout& L, const tq_prob_dev& P, int x_type,
                                hipStream_t stream);
tq_status tq_gemv_launch_grouped(int family, int waves, int row_blocks, const void* workspace,
                                 int64_t n_probs, int64_t n_items, int x_lds_bytes, hipStream_t stream);
// The same with one item per wave: `wave_items` items, `waves` per workgroup
// (bf16, no column split, no codebook).
tq_status tq_gemv_launch_wave_items(int family, int waves, const void* workspace, int64_t n_probs,
                                    int64_t wave_items, hipStream_t stream);
// Bytes of one activation element as the decode kernels read x.
static inline int64_t tq_x_elem_bytes(int x_type)
{
    return x_type == TQ_BF16 ? 2 : (x_type == TQ_I8 ? 1 : 4);
}
// Tokens m0 .. m0 + m - 1 of a problem, as a problem of their own.
static inline tq_prob_dev tq_prob_slice(const tq_prob_dev& P, int x_type, int m0, int m)
{
    tq_prob_dev Q = P;
    Q.x = P.x ? (const uint8_t*)P.x + (int64_t)m0 * P.Kin * tq_x_elem_bytes(x_type) : nullptr;
    Q.x_scale = P.x_scale ? P.x_scale + m0 : nullptr;
    Q.y = P.y ? P.y + (int64_t)m0 * P.N : nullptr;
    Q.acc = P.acc ? P.acc + (int64_t)m0 * P.N : nullptr;
    Q.M = m;
    return Q;
}
// LDS bytes of M tokens x Kin int8 activations (TQ_F32_Q8), 16-byte rounded.
static inline size_t tq_x_lds_bytes(int64_t M, int64_t Kin) { return (size_t)((M * Kin + 15) & ~(int64_t)15); }
// Workspace layout of a grouped plan: problem table, then the items.
static inline int64_t tq_ws_items_off(int64_t n_probs) { return tq_align256(n_probs * (int64_t)sizeof(tq_prob_dev)); }
#define TQ_MAX_Q8_LDS 65536
// LDS of one workgroup on gfx950, and what a decode launch asks for: the
// kernel's static arrays (the bf16 trit table; 1 KiB covers the small ones),
// the partial sums of split row blocks and the int8 copy of x.
#define TQ_MAX_WG_LDS 163840
size_t tq_gemv_lds_bytes(int family, int split_waves, int total_waves, size_t x_lds_bytes);
// Family id of a (x_type, layout, K, M) combination, or -1 if none.
int tq_gemv_family(int x_type, int layout, int K, int M);
