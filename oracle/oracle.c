/*
 * CPU oracle of the packed ternary-weight product -- TEST INFRASTRUCTURE.
 *
 * Only the tests, the package's smoke check and the benchmark's CPU-baseline
 * leg load this library.  It shares no code, header, table or helper with the
 * HIP library; it sees only the canonical (unpacked) arrays.
 *
 * What it computes is the definition written out as plain loops:
 *
 *   y[m][n] = sum_k sum_g S_k[n][g] * sum_{i in group g} t_k[n][i] * x[m][i]
 *
 * - The weight is a base plane of values -1, 0, +1 plus residual planes of
 *   the same kind (Tritium page, introduction): planes are summed, plane 0
 *   first.
 * - Each plane is scaled group by group before the planes are added, with
 *   one f16 scale per plane per group of g weights along the row (sasori
 *   page, "How it works" and the
 *   "K and g" table, whose bits-per-weight figures 2K + 16K/g only add up
 *   with one f16 per plane per group).
 * - A per-tensor scale applied once at the end ("Ternary GEMV (No
 *   Multiplication)" section of the QORA-LLM-2B page).
 * - The balanced-ternary codec: d = 3 digits give 27 levels, value
 *   9 t2 + 3 t1 + t0, groups of 16 weights whose scale is one of 27
 *   log-spaced f16 values
 *   (Llama-3.1-8B-trit-uniform-d3 card, "Quantization details").  Plane p
 *   carries the digit of weight 3^(K-1-p), so S_p[n][g] = 3^(K-1-p) cb[idx].
 * - The result equals the dense product with the dequantised weight, the
 *   fake-quant result that the sasori kernel is said to match bit for bit (sasori page,
 *   "g (group-size)") and the FP16-dequantised checkpoint of the model card
 *   ("Quick load").
 *
 * Floating-point paths accumulate in fp64 after converting every input
 * exactly (bf16 -> fp32 -> fp64, f16 -> fp64).  The int8-activation path
 * follows the per-token absmax quantiser and the integer accumulate exactly,
 * and for one plane with a per-tensor scale produces the fp32 result with the
 * two fp32 multiplies in the stated order.  Build with -O2
 * -ffp-contract=off and no fast-math so that the fp32 steps are single IEEE
 * operations.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_OK = 0, OR_ERR_ARG = 1, OR_ERR_SHAPE = 2, OR_ERR_VALUE = 4 };
enum { OR_TENSOR = 0, OR_GROUP_F16 = 1, OR_CODEBOOK = 2 };
enum { OR_F32 = 0, OR_BF16 = 1, OR_I8 = 2 };

/* IEEE 754 binary16 -> double, from the format's definition. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int exp = (h >> 10) & 0x1F;
    int frac = h & 0x3FF;
    double v;
    if (exp == 0)
        v = ldexp((double)frac, -24);            /* subnormal: frac * 2^-24 */
    else if (exp == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), exp - 25); /* 1.frac * 2^(exp-15) */
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
float oracle_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static double x_value(int x_type, const void* x, int64_t idx)
{
    if (x_type == OR_BF16)
        return (double)oracle_bf16_to_f32(((const uint16_t*)x)[idx]);
    return (double)((const float*)x)[idx];
}

static int check_desc(int K, int g, int layout, int n_cb, int64_t N, int64_t Kin)
{
    if (K < 1 || K > 4 || N < 0 || Kin < 0) return OR_ERR_ARG;
    if (layout == OR_TENSOR) return OR_OK;
    if (layout != OR_GROUP_F16 && layout != OR_CODEBOOK) return OR_ERR_ARG;
    if (g <= 0 || Kin % g != 0) return OR_ERR_SHAPE;
    if (layout == OR_CODEBOOK && (n_cb < 1 || n_cb > 32)) return OR_ERR_ARG;
    return OR_OK;
}

/* The scale S_k[n][g] of the definition, as an exact fp64 value. */
static double scale_of(int layout, int K, int k, int64_t n, int64_t G, int64_t grp,
                       const void* scales, const uint16_t* codebook, int64_t N)
{
    if (layout == OR_TENSOR)
        return (double)((const float*)scales)[k];
    if (layout == OR_GROUP_F16)
        return oracle_f16_to_f64(((const uint16_t*)scales)[((int64_t)k * N + n) * G + grp]);
    /* codebook: plane k is digit weight 3^(K-1-k) */
    {
        double w = 1.0;
        int j;
        uint8_t idx = ((const uint8_t*)scales)[n * G + grp];
        for (j = 0; j < K - 1 - k; ++j) w *= 3.0;
        return w * oracle_f16_to_f64(codebook[idx]);
    }
}

static int check_values(int K, int layout, int n_cb, int64_t N, int64_t Kin, int64_t G,
                        const int8_t* trits, const void* scales, const uint16_t* codebook)
{
    int64_t i, total = (int64_t)K * N * Kin;
    for (i = 0; i < total; ++i)
        if (trits[i] < -1 || trits[i] > 1) return OR_ERR_VALUE;
    if (layout == OR_TENSOR) {
        for (i = 0; i < K; ++i)
            if (!isfinite(((const float*)scales)[i])) return OR_ERR_VALUE;
    } else if (layout == OR_GROUP_F16) {
        for (i = 0; i < (int64_t)K * N * G; ++i)
            if (!isfinite(oracle_f16_to_f64(((const uint16_t*)scales)[i]))) return OR_ERR_VALUE;
    } else {
        for (i = 0; i < N * G; ++i)
            if (((const uint8_t*)scales)[i] >= n_cb) return OR_ERR_VALUE;
        for (i = 0; i < n_cb; ++i)
            if (!isfinite(oracle_f16_to_f64(codebook[i]))) return OR_ERR_VALUE;
    }
    return OR_OK;
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Floating-point activations (fp32, or bf16 bits).  y is fp64 [M][N].
 */
int oracle_gemv_fp(int K, int g, int layout, int n_cb, int64_t N, int64_t Kin,
                   const int8_t* trits, const void* scales, const uint16_t* codebook,
                   int64_t M, int x_type, const void* x, double* y, int nthreads)
{
    int64_t G, gs, m, i;
    int rc = check_desc(K, g, layout, n_cb, N, Kin);
    if (rc) return rc;
    if (x_type != OR_F32 && x_type != OR_BF16) return OR_ERR_ARG;
    if (M < 0) return OR_ERR_ARG;
    gs = (layout == OR_TENSOR) ? (Kin > 0 ? Kin : 1) : g;  /* per-tensor: one group per row */
    G = (layout == OR_TENSOR) ? 1 : Kin / g;
    rc = check_values(K, layout, n_cb, N, Kin, G, trits, scales, codebook);
    if (rc) return rc;
    for (i = 0; i < M * Kin; ++i)
        if (!isfinite(x_value(x_type, x, i))) return OR_ERR_VALUE;
    set_threads(nthreads);
    for (m = 0; m < M; ++m) {
        int64_t n;
#pragma omp parallel for schedule(static)
        for (n = 0; n < N; ++n) {
            double acc = 0.0;
            int k;
            for (k = 0; k < K; ++k) {
                int64_t grp;
                for (grp = 0; grp < G; ++grp) {
                    double p = 0.0;   /* sum over the group: +x, -x or nothing */
                    int64_t j;
                    for (j = grp * gs; j < (grp + 1) * gs && j < Kin; ++j) {
                        int8_t t = trits[((int64_t)k * N + n) * Kin + j];
                        double xv = x_value(x_type, x, m * Kin + j);
                        if (t == 1) p += xv;
                        else if (t == -1) p -= xv;
                    }
                    acc += scale_of(layout, K, k, n, G, grp, scales, codebook, N) * p;
                }
            }
            y[m * N + n] = acc;
        }
    }
    return OR_OK;
}

/*
 * Per-token absmax int8 quantisation, in fp32:
 *   a = max_i |x_i|;  a == 0 -> q = 0, s = 0;
 *   inv = fl(127 / a);  q_i = clamp(rint(fl(x_i * inv)), -127, 127);  s = fl(a / 127).
 */
int oracle_act_quant_i8(int64_t M, int64_t Kin, int x_type, const void* x,
                        int8_t* q, float* s)
{
    int64_t m, i;
    if (M < 0 || Kin < 0) return OR_ERR_ARG;
    if (x_type != OR_F32 && x_type != OR_BF16) return OR_ERR_ARG;
    for (m = 0; m < M; ++m) {
        float a = 0.0f, inv;
        for (i = 0; i < Kin; ++i) {
            float v = (float)x_value(x_type, x, m * Kin + i);
            if (!isfinite(v)) return OR_ERR_VALUE;
            if (fabsf(v) > a) a = fabsf(v);
        }
        if (a == 0.0f) {
            for (i = 0; i < Kin; ++i) q[m * Kin + i] = 0;
            s[m] = 0.0f;
            continue;
        }
        inv = 127.0f / a;
        for (i = 0; i < Kin; ++i) {
            float v = (float)x_value(x_type, x, m * Kin + i);
            float r = rintf(v * inv);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            q[m * Kin + i] = (int8_t)r;
        }
        s[m] = a / 127.0f;
    }
    return OR_OK;
}

/*
 * int8 activations with their per-token scales.
 *   acc_kg = sum_{i in g} t_k[n][i] * q[m][i]          (exact integers)
 *   acc[m][n] = sum_k sum_g acc_kg                      (int64, written if acc != 0)
 *   y64[m][n] = sum_k sum_g S_k[n][g] * acc_kg * s_x[m] (fp64, written if y64 != 0)
 *   y32[m][n] (one plane, per-tensor scale only) = fl(float(acc) * fl(s_w * s_x[m]))
 */
int oracle_gemv_i8(int K, int g, int layout, int n_cb, int64_t N, int64_t Kin,
                   const int8_t* trits, const void* scales, const uint16_t* codebook,
                   int64_t M, const int8_t* xq, const float* xs,
                   int64_t* acc, double* y64, float* y32, int nthreads)
{
    int64_t G, gs, m;
    int rc = check_desc(K, g, layout, n_cb, N, Kin);
    if (rc) return rc;
    if (M < 0) return OR_ERR_ARG;
    if (y32 && !(layout == OR_TENSOR && K == 1)) return OR_ERR_ARG;
    gs = (layout == OR_TENSOR) ? (Kin > 0 ? Kin : 1) : g;
    G = (layout == OR_TENSOR) ? 1 : Kin / g;
    rc = check_values(K, layout, n_cb, N, Kin, G, trits, scales, codebook);
    if (rc) return rc;
    set_threads(nthreads);
    for (m = 0; m < M; ++m) {
        int64_t n;
#pragma omp parallel for schedule(static)
        for (n = 0; n < N; ++n) {
            int64_t total = 0;
            double yacc = 0.0;
            int k;
            for (k = 0; k < K; ++k) {
                int64_t grp;
                for (grp = 0; grp < G; ++grp) {
                    int64_t p = 0, j;
                    for (j = grp * gs; j < (grp + 1) * gs && j < Kin; ++j) {
                        int8_t t = trits[((int64_t)k * N + n) * Kin + j];
                        int64_t xv = xq[m * Kin + j];
                        if (t == 1) p += xv;
                        else if (t == -1) p -= xv;
                    }
                    total += p;
                    yacc += scale_of(layout, K, k, n, G, grp, scales, codebook, N) * (double)p
                            * (double)xs[m];
                }
            }
            if (acc) acc[m * N + n] = total;
            if (y64) y64[m * N + n] = yacc;
            if (y32) {
                float c = ((const float*)scales)[0] * xs[m];   /* fl(s_w * s_x) */
                y32[m * N + n] = (float)total * c;              /* fl(float(acc) * c) */
            }
        }
    }
    return OR_OK;
}
