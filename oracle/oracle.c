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
#include <stdlib.h>
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

/* ------------------------------------------------------------------------
 * One BitNet b1.58 layer as a decode chain for one token (QORA-LLM-2B page,
 * "SubLN Pattern" listing, and its "Architecture" table for the head
 * counts): every ternary linear takes its input quantised to int8 per token
 * (the int8 path above, one plane and a per-tensor scale), and the steps run
 * in the listing's order.
 * ------------------------------------------------------------------------ */

/*
 * RMSNorm (the listing's input, attention-sub, post-attention and FFN-sub
 * norms): out_i = x_i / sqrt(mean(x^2) + eps) * w_i.  The sum of squares is
 * taken in fp64 (each square exact), the mean rounded once to fp32, and the
 * rest is single fp32 operations:
 *   ms = fl32(ss / n);  r = fl(1 / fl(sqrt(fl(ms + eps))));  out_i = fl(fl(x_i * r) * w_i).
 */
int oracle_rms_norm(int64_t n, const float* x, const float* w, float eps, float* out)
{
    int64_t i;
    double ss = 0.0;
    float ms, r;
    if (n <= 0 || !x || !w || !out) return OR_ERR_ARG;
    for (i = 0; i < n; ++i) {
        if (!isfinite(x[i]) || !isfinite(w[i])) return OR_ERR_VALUE;
        ss += (double)x[i] * (double)x[i];
    }
    ms = (float)(ss / (double)n);
    r = 1.0f / sqrtf(ms + eps);
    for (i = 0; i < n; ++i) out[i] = (x[i] * r) * w[i];
    return OR_OK;
}

/* The FFN's squared-ReLU gate times the up projection (same listing):
 * out_i = fl(fl(g'_i * g'_i) * u_i) with g'_i = max(0, g_i). */
int oracle_relu2_mul(int64_t n, const float* g, const float* u, float* out)
{
    int64_t i;
    if (n < 0 || (n > 0 && (!g || !u || !out))) return OR_ERR_ARG;
    for (i = 0; i < n; ++i) {
        float a = g[i] > 0.0f ? g[i] : 0.0f;
        out[i] = (a * a) * u[i];
    }
    return OR_OK;
}

/* y = fl32 result of one ternary linear (one plane, per-tensor scale s_w) on
 * the int8 quantisation of x: the int8 path above. */
static int linear_i8(int64_t N, int64_t Kin, const int8_t* trits, float s_w, const float* x,
                     float* y, int8_t* q_tmp)
{
    float sx;
    int rc = oracle_act_quant_i8(1, Kin, OR_F32, x, q_tmp, &sx);
    if (rc) return rc;
    return oracle_gemv_i8(1, 0, OR_TENSOR, 0, N, Kin, trits, &s_w, 0, 1, q_tmp, &sx, 0, 0, y, 0);
}

/*
 * One layer for the first token of a sequence (position 0).  With a single
 * cached key the attention softmax has one weight, 1, so each query head's
 * output is the value vector of its KV head: query head h reads KV head
 * h / (n_heads / n_kv), the consecutive grouping of grouped-query attention.
 * RoPE, q and k then leave the output unchanged; q, k and v are still
 * computed and returned (qkv), as a decode step stores k and v.
 *
 *   h  = RMSNorm(x, w_in);            q, k, v = W_q h, W_k h, W_v h
 *   a  = repeat(v);  a = RMSNorm(a, w_attn_sub);  x1 = x + W_o a
 *   h2 = RMSNorm(x1, w_post);         g, u = W_gate h2, W_up h2
 *   f  = RMSNorm(relu2(g) * u, w_ffn_sub);  x <- x1 + W_down f
 *
 * trits[p], s_w[p]: projection p in the order q, k, v, o, gate, up, down,
 * int8 [N][Kin] and its per-tensor scale.  x: [hidden], updated in place.
 * qkv (optional): [(n_heads + 2 n_kv) * head_dim], q then k then v.
 */
int oracle_bitnet_layer(int64_t hidden, int64_t inter, int n_heads, int n_kv, int head_dim, float eps,
                        const int8_t* const* trits, const float* s_w, const float* w_in,
                        const float* w_attn_sub, const float* w_post, const float* w_ffn_sub,
                        float* x, float* qkv)
{
    const int64_t nq = (int64_t)n_heads * head_dim, nkv = (int64_t)n_kv * head_dim;
    const int64_t big = hidden > inter ? (hidden > nq ? hidden : nq) : (inter > nq ? inter : nq);
    int64_t i;
    int rc = OR_OK;
    float *h, *q, *k, *v, *a, *o, *x1, *g, *u, *f, *d;
    int8_t* qt;
    if (hidden <= 0 || inter <= 0 || n_heads <= 0 || n_kv <= 0 || head_dim <= 0) return OR_ERR_ARG;
    if (n_heads % n_kv != 0 || nq != hidden) return OR_ERR_SHAPE;
    h = (float*)malloc(sizeof(float) * (size_t)(big * 8 + nq + 2 * nkv));
    qt = (int8_t*)malloc((size_t)big);
    if (!h || !qt) {
        free(h);
        free(qt);
        return OR_ERR_ARG;
    }
    q = h + big; k = q + nq; v = k + nkv; a = v + nkv; o = a + big; x1 = o + big;
    g = x1 + big; u = g + big; f = u + big; d = f + big;

    if ((rc = oracle_rms_norm(hidden, x, w_in, eps, h))) goto done;
    if ((rc = linear_i8(nq, hidden, trits[0], s_w[0], h, q, qt))) goto done;
    if ((rc = linear_i8(nkv, hidden, trits[1], s_w[1], h, k, qt))) goto done;
    if ((rc = linear_i8(nkv, hidden, trits[2], s_w[2], h, v, qt))) goto done;
    for (i = 0; i < nq; ++i) {
        const int64_t head = i / head_dim, kvh = head / (n_heads / n_kv);
        a[i] = v[kvh * head_dim + i % head_dim];
    }
    if ((rc = oracle_rms_norm(nq, a, w_attn_sub, eps, a))) goto done;
    if ((rc = linear_i8(hidden, nq, trits[3], s_w[3], a, o, qt))) goto done;
    for (i = 0; i < hidden; ++i) x1[i] = x[i] + o[i];
    if ((rc = oracle_rms_norm(hidden, x1, w_post, eps, h))) goto done;
    if ((rc = linear_i8(inter, hidden, trits[4], s_w[4], h, g, qt))) goto done;
    if ((rc = linear_i8(inter, hidden, trits[5], s_w[5], h, u, qt))) goto done;
    if ((rc = oracle_relu2_mul(inter, g, u, f))) goto done;
    if ((rc = oracle_rms_norm(inter, f, w_ffn_sub, eps, f))) goto done;
    if ((rc = linear_i8(hidden, inter, trits[6], s_w[6], f, d, qt))) goto done;
    for (i = 0; i < hidden; ++i) x[i] = x1[i] + d[i];
    if (qkv) memcpy(qkv, q, sizeof(float) * (size_t)(nq + 2 * nkv));
done:
    free(h);
    free(qt);
    return rc;
}

/* ------------------------------------------------------------------------
 * Ternarizer: the step before packing -- a dense weight fit into K trit
 * planes (sasori page, "How it works & paper": each matrix is fit on its
 * own into a sum of K per-group-scaled trit-planes, weight-only) or into
 * the balanced-ternary codec (d3 card, "Quantization details": uniform
 * post-training quantisation, 27 levels, groups of 16, a 27-entry
 * log-spaced scale codebook).
 * ------------------------------------------------------------------------ */

/* fp32 -> IEEE binary16 bits, round to nearest even; magnitudes above the
 * largest finite half saturate to it (65504). */
uint16_t oracle_f32_to_f16(float f)
{
    double a = fabs((double)f);
    uint16_t sign = signbit(f) ? 0x8000u : 0u;
    int e;
    double m, q;
    uint32_t bits;
    if (a >= 65504.0) return (uint16_t)(sign | 0x7BFFu);
    if (a < ldexp(1.0, -24) * 0.5) return sign;              /* rounds to zero (ties to even) */
    e = (int)floor(log2(a));
    if (ldexp(1.0, e) > a) e -= 1;                             /* guard the log */
    if (ldexp(1.0, e + 1) <= a) e += 1;
    if (e < -14) {                                             /* subnormal: multiples of 2^-24 */
        q = nearbyint(a / ldexp(1.0, -24));
        return (uint16_t)(sign | (uint16_t)q);
    }
    m = a / ldexp(1.0, e);                                     /* in [1, 2) */
    q = nearbyint((m - 1.0) * 1024.0);                         /* 10 mantissa bits, ties to even */
    if (q == 1024.0) {
        q = 0.0;
        e += 1;
    }
    if (e > 15) return (uint16_t)(sign | 0x7BFFu);
    bits = ((uint32_t)(e + 15) << 10) | (uint32_t)q;
    return (uint16_t)(sign | bits);
}

/* The balanced-ternary digits of q in [-(3^K - 1)/2, (3^K - 1)/2]: q =
 * sum_d 3^d t_d with t_d in {-1, 0, 1}; digit d written to dig[d]. */
static void balanced_digits(int q, int K, int8_t* dig)
{
    int d;
    for (d = 0; d < K; ++d) {
        int r = ((q % 3) + 3) % 3;                /* 0, 1, 2 */
        int t = r == 2 ? -1 : r;
        dig[d] = (int8_t)t;
        q = (q - t) / 3;
    }
}

/*
 * Fit w [N][Kin] (fp32) into trits [K][N][Kin] and canonical scales.
 *
 * TQ_SCALE_GROUP_F16 and TQ_SCALE_TENSOR -- greedy residual planes:
 *   R = w;  for k = 0 .. K-1, per group (g consecutive inputs of a row; the
 *   whole tensor for TENSOR):
 *     a = mean |R| over the group                  (the absmean of BitNet b1.58)
 *     t = sign(R) where |R| > a / 2, else 0         (round(R / a) clipped to
 *                                                    [-1, 1], as an exact
 *                                                    comparison)
 *     s = mean |R| over the entries with t != 0     (the least-squares scale
 *                                                    of the plane t; 0 if none)
 *     R = fl(R - s t)
 *   Sums are fp64 (row by row in index order; for TENSOR the row sums then
 *   added in row order), divided in fp64 and rounded to fp32; s is then
 *   rounded to f16 for GROUP_F16 (ties to even, saturating at 65504), and
 *   the rounded s is what the residual uses.  A plane never increases a
 *   group's squared error (s is optimal for t, and s = 0 would leave it).
 *
 * TQ_SCALE_CODEBOOK -- uniform quantisation onto L = (3^K - 1) / 2 levels a
 * side with a scale from the codebook (ascending) per group:
 *   a = max |w|;  c = fl(a / L);  idx = the first entry with cb[idx] >= c
 *   (the last if none);  q = clamp(rint(fl(w / cb[idx])), -L, L);
 *   digits of q in balanced ternary, plane p holding the digit of 3^(K-1-p).
 */
int oracle_ternarize(int K, int g, int layout, int n_cb, int64_t N, int64_t Kin, const float* w,
                     const uint16_t* codebook, int8_t* trits, void* scales)
{
    int64_t n, i, G;
    int rc = check_desc(K, g, layout, n_cb, N, Kin);
    if (rc) return rc;
    for (i = 0; i < N * Kin; ++i)
        if (!isfinite(w[i])) return OR_ERR_VALUE;
    if (layout == OR_CODEBOOK) {
        const int L = (K == 1) ? 1 : (K == 2 ? 4 : (K == 3 ? 13 : 40));
        int j;
        for (j = 0; j + 1 < n_cb; ++j)
            if (!(oracle_f16_to_f64(codebook[j]) < oracle_f16_to_f64(codebook[j + 1]))) return OR_ERR_VALUE;
        if (!(oracle_f16_to_f64(codebook[0]) > 0.0)) return OR_ERR_VALUE;
        G = Kin / g;
        for (n = 0; n < N; ++n) {
            int64_t grp;
            for (grp = 0; grp < G; ++grp) {
                float a = 0.0f, c, s;
                int idx = n_cb - 1;
                for (i = grp * g; i < (grp + 1) * g; ++i)
                    if (fabsf(w[n * Kin + i]) > a) a = fabsf(w[n * Kin + i]);
                c = a / (float)L;
                for (j = 0; j < n_cb; ++j) {
                    if ((float)oracle_f16_to_f64(codebook[j]) >= c) {
                        idx = j;
                        break;
                    }
                }
                ((uint8_t*)scales)[n * G + grp] = (uint8_t)idx;
                s = (float)oracle_f16_to_f64(codebook[idx]);
                for (i = grp * g; i < (grp + 1) * g; ++i) {
                    float q = rintf(w[n * Kin + i] / s);
                    int8_t dig[4];
                    int p;
                    if (q > (float)L) q = (float)L;
                    if (q < -(float)L) q = -(float)L;
                    balanced_digits((int)q, K, dig);
                    for (p = 0; p < K; ++p) trits[((int64_t)p * N + n) * Kin + i] = dig[K - 1 - p];
                }
            }
        }
        return OR_OK;
    }
    {
        float* R = (float*)malloc(sizeof(float) * (size_t)(N * Kin));
        double* rowsum = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        int k;
        const int64_t gs = layout == OR_TENSOR ? Kin : g;
        if (!R || !rowsum) {
            free(R);
            free(rowsum);
            return OR_ERR_ARG;
        }
        G = layout == OR_TENSOR ? 1 : Kin / g;
        memcpy(R, w, sizeof(float) * (size_t)(N * Kin));
        for (k = 0; k < K; ++k) {
            /* per group: the absmean a, the plane t, then its scale s */
            for (n = 0; n < N; ++n) {
                int64_t grp;
                for (grp = 0; grp < G; ++grp) {
                    double sum = 0.0, sum_nz = 0.0;
                    int64_t nz = 0;
                    float a, sc;
                    if (layout == OR_TENSOR) break;
                    for (i = grp * gs; i < (grp + 1) * gs; ++i) sum += fabs((double)R[n * Kin + i]);
                    a = (float)(sum / (double)gs);
                    for (i = grp * gs; i < (grp + 1) * gs; ++i) {
                        float t = 0.0f;
                        if (a > 0.0f && fabsf(R[n * Kin + i]) > 0.5f * a) t = R[n * Kin + i] > 0.0f ? 1.0f : -1.0f;
                        trits[((int64_t)k * N + n) * Kin + i] = (int8_t)t;
                        if (t != 0.0f) {
                            sum_nz += fabs((double)R[n * Kin + i]);
                            nz += 1;
                        }
                    }
                    sc = nz > 0 ? (float)(sum_nz / (double)nz) : 0.0f;
                    {
                        const uint16_t h = oracle_f32_to_f16(sc);
                        ((uint16_t*)scales)[((int64_t)k * N + n) * G + grp] = h;
                        sc = (float)oracle_f16_to_f64(h);
                    }
                    for (i = grp * gs; i < (grp + 1) * gs; ++i)
                        R[n * Kin + i] = R[n * Kin + i] - sc * (float)trits[((int64_t)k * N + n) * Kin + i];
                }
            }
            if (layout == OR_TENSOR) {
                double tot = 0.0, tot_nz = 0.0;
                int64_t nz = 0;
                float a, sc;
                for (n = 0; n < N; ++n) {
                    double sr = 0.0;
                    for (i = 0; i < Kin; ++i) sr += fabs((double)R[n * Kin + i]);
                    rowsum[n] = sr;
                }
                for (n = 0; n < N; ++n) tot += rowsum[n];
                a = (N * Kin > 0) ? (float)(tot / (double)(N * Kin)) : 0.0f;
                for (n = 0; n < N; ++n) {
                    double sr = 0.0;
                    for (i = 0; i < Kin; ++i) {
                        float t = 0.0f;
                        if (a > 0.0f && fabsf(R[n * Kin + i]) > 0.5f * a) t = R[n * Kin + i] > 0.0f ? 1.0f : -1.0f;
                        trits[((int64_t)k * N + n) * Kin + i] = (int8_t)t;
                        if (t != 0.0f) {
                            sr += fabs((double)R[n * Kin + i]);
                            nz += 1;
                        }
                    }
                    rowsum[n] = sr;
                }
                for (n = 0; n < N; ++n) tot_nz += rowsum[n];
                sc = nz > 0 ? (float)(tot_nz / (double)nz) : 0.0f;
                ((float*)scales)[k] = sc;
                for (i = 0; i < N * Kin; ++i) R[i] = R[i] - sc * (float)trits[(int64_t)k * N * Kin + i];
            }
        }
        free(R);
        free(rowsum);
    }
    return OR_OK;
}
