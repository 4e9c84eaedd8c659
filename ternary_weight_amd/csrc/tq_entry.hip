// libtq: tq_gemv, tq_gemv_grouped_* entry points (validation and dispatch).
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "tq_internal.h"

static int log2i(int v)
{
    int r = 0;
    while ((1 << r) < v) ++r;
    return r;
}

// Prefix the thread's last error message with the problem index.
tq_status tq_fail_problem(tq_status s, int32_t i)
{
    char msg[512];
    snprintf(msg, sizeof msg, "%s", tq_last_error());
    return tq_fail(s, "problem %d: %s", (int)i, msg);
}

static bool acc_allowed(const tq_layout& L, int x_type)
{
    return (x_type == TQ_I8 || x_type == TQ_F32_Q8) && L.layout == TQ_SCALE_TENSOR && L.K == 1;
}

tq_status tq_check_call(const tq_layout& L, const void* blob, int64_t M, int32_t x_type, const void* x,
                        const float* x_scale, const float* y, const int32_t* acc, int64_t max_m,
                        int x_align)
{
    tq_status s;
    if (x_type != TQ_F32 && x_type != TQ_BF16 && x_type != TQ_I8 && x_type != TQ_F32_Q8)
        return tq_fail(TQ_ERR_ARG, "x_type = %d is not a tq_dtype", x_type);
    if (M < 0) return tq_fail(TQ_ERR_ARG, "M = %lld is negative", (long long)M);
    if (M > max_m) return tq_fail(TQ_ERR_UNSUPPORTED, "M = %lld exceeds %lld for this call",
                                  (long long)M, (long long)max_m);
    const bool work = M > 0 && L.N > 0;
    if ((s = tq_check_ptr(blob, "blob", !work))) return s;
    if ((s = tq_check_ptr(x, "x", !(work && L.Kin > 0), x_type == TQ_F32_Q8 ? 16 : x_align))) return s;
    if (x_type == TQ_F32_Q8 && (int64_t)tq_x_lds_bytes(M, L.Kin) > TQ_MAX_Q8_LDS)
        return tq_fail(TQ_ERR_UNSUPPORTED, "TQ_F32_Q8 needs M * in_features <= %d (LDS); got %lld",
                       TQ_MAX_Q8_LDS, (long long)(M * L.Kin));
    if ((s = tq_check_ptr(y, "y", !work, 4))) return s;
    if (x_type == TQ_I8) {
        if ((s = tq_check_ptr(x_scale, "x_scale", !work, 4))) return s;
    }
    if (acc) {
        if (!acc_allowed(L, x_type))
            return tq_fail(TQ_ERR_UNSUPPORTED,
                           "acc output needs int8 activations, TQ_SCALE_TENSOR and one plane");
        if ((s = tq_check_ptr(acc, "acc", true, 4))) return s;
    }
    return TQ_OK;
}

tq_prob_dev tq_make_prob(const tq_layout& L, const void* blob, int64_t M, const void* x,
                      const float* x_scale, float* y, int32_t* acc)
{
    tq_prob_dev P;
    memset(&P, 0, sizeof P);
    const uint8_t* b = (const uint8_t*)blob;
    P.codes = b + L.codes_off;
    P.scales = b + L.scales_off;
    P.cb = L.layout == TQ_SCALE_CODEBOOK ? (const uint16_t*)(b + L.cb_off) : nullptr;
    P.x = x;
    P.x_scale = x_scale;
    P.y = y;
    P.acc = acc;
    P.N = (int32_t)L.N;
    P.Kin = (int32_t)L.Kin;
    P.NC = (int32_t)L.NC;
    P.NGD = (int32_t)L.NGD;
    P.NID = (int32_t)L.NID;
    P.g = L.layout == TQ_SCALE_TENSOR ? 0 : L.g;
    P.M = (int32_t)M;
    P.log2g = L.layout == TQ_SCALE_TENSOR ? 0 : log2i(L.g);
    return P;
}


TQ_EXPORT tq_status tq_gemv(const tq_weight_desc* desc, const void* blob, int64_t M, int32_t x_type,
                            const void* x, const float* x_scale, float* y, int32_t* acc, void* stream)
{
    tq_layout L;
    tq_status s = tq_check_desc(desc, &L);
    if (s) return s;
    if ((s = tq_check_call(L, blob, M, x_type, x, x_scale, y, acc, TQ_MAX_M_GEMV))) return s;
    if (M == 0 || L.N == 0) return tq_ok();
    const tq_prob_dev P = tq_make_prob(L, blob, M, x, x_scale, y, acc);
    if (tq_gemv_uses_mfma(x_type, M, x))
        s = tq_gemm_launch(L, P, x_type, (hipStream_t)stream);
    else
        s = tq_gemv_launch_single(L, P, x_type, (hipStream_t)stream);
    if (s) return s;
    return tq_ok();
}

TQ_EXPORT tq_status tq_gemv_grouped_workspace_size(const tq_problem* problems, int32_t count,
                                                   int64_t M, size_t* bytes)
{
    if (!bytes) return tq_fail(TQ_ERR_ARG, "bytes is NULL");
    if (count < 0 || (count > 0 && !problems)) return tq_fail(TQ_ERR_ARG, "bad problem list");
    if (M < 0 || M > TQ_MAX_M_GEMV) return tq_fail(TQ_ERR_UNSUPPORTED, "M = %lld not in 0..%d",
                                                   (long long)M, TQ_MAX_M_GEMV);
    int64_t items = 0;
    for (int32_t i = 0; i < count; ++i) {
        tq_layout L;
        tq_status s = tq_check_desc(problems[i].desc, &L);
        if (s) return tq_fail_problem(s, i);
        items += L.NB;
    }
    // problems, then one (problem, first row block) item per workgroup (at most one per block)
    *bytes = (size_t)(tq_ws_items_off(count) + tq_align256(items * 8));
    if (*bytes == 0) *bytes = 256;
    return tq_ok();
}

TQ_EXPORT tq_status tq_gemv_grouped_prepare(const tq_problem* problems, int32_t count, int64_t M,
                                            int32_t x_type, void* workspace, size_t workspace_bytes,
                                            tq_grouped_plan* plan, void* stream)
{
    if (!plan) return tq_fail(TQ_ERR_ARG, "plan is NULL");
    const int pow2[] = {1, 2, 4, 8, 16};
    auto is_shape = [&](int v) { for (int p : pow2) if (v == p) return true; return false; };
    int waves = plan->waves, row_blocks = plan->row_blocks;
    const bool hinted = is_shape(waves) && is_shape(row_blocks) && waves * row_blocks <= 16;
    if (!hinted) {
        // bf16: the trit table fills 64 KiB of LDS, so 16 one-wave row blocks share it
        waves = (x_type == TQ_F32_Q8 || x_type == TQ_BF16) ? 1 : 4;
        row_blocks = x_type == TQ_F32_Q8 ? 4 : (x_type == TQ_BF16 ? 16 : 1);
    }
    size_t need = 0;
    tq_status s = tq_gemv_grouped_workspace_size(problems, count, M, &need);
    if (s) return s;
    // several bf16 tokens: the matrix-core kernels, if every x allows 16-byte loads
    bool mfma = count > 0;
    for (int32_t i = 0; i < count; ++i) mfma = mfma && tq_gemv_uses_mfma(x_type, M, problems[i].x);
    if (mfma) return tq_gemm_grouped_prepare(problems, count, M, x_type, workspace, workspace_bytes, plan, stream);
    if ((s = tq_check_ptr(workspace, "workspace", false))) return s;
    if (workspace_bytes < need)
        return tq_fail(TQ_ERR_ARG, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    std::vector<tq_prob_dev> probs((size_t)count);
    struct Item { int64_t cost; int32_t prob, rb0; };
    std::vector<Item> items;
    int family = -1, K0 = 0, layout0 = -1, g0 = 0;
    size_t x_lds = 0;
    for (int32_t i = 0; i < count; ++i) {
        const tq_problem& pr = problems[i];
        tq_layout L;
        tq_check_desc(pr.desc, &L);
        if ((s = tq_check_call(L, pr.blob, M, x_type, pr.x, pr.x_scale, pr.y, pr.acc, TQ_MAX_M_GEMV)))
            return tq_fail_problem(s, i);
        if (i == 0) {
            K0 = L.K;
            layout0 = L.layout;
            g0 = L.g;
        } else if (L.K != K0 || L.layout != layout0 || (L.layout != TQ_SCALE_TENSOR && L.g != g0)) {
            return tq_fail(TQ_ERR_UNSUPPORTED,
                           "problem %d: all problems of a plan must share planes, layout and group", i);
        }
        probs[(size_t)i] = tq_make_prob(L, pr.blob, M, pr.x, pr.x_scale, pr.y, pr.acc);
        if (x_type == TQ_F32_Q8) x_lds = std::max(x_lds, tq_x_lds_bytes(M, L.Kin));
    }
    if (count > 0 && M > 0) {
        family = tq_gemv_family(x_type, layout0, K0, (int)M);
        // a shape whose partial sums overflow the workgroup's LDS: the default
        // one gives up the column split first, a requested one is refused
        auto lds = [&](int w, int rbs) { return tq_gemv_lds_bytes(family, w, w * rbs, x_lds); };
        if (lds(waves, row_blocks) > TQ_MAX_WG_LDS) {
            if (hinted) return tq_fail(TQ_ERR_UNSUPPORTED, "plan shape %d x %d needs more LDS than a "
                                       "workgroup has", waves, row_blocks);
            while (waves > 1 && lds(waves, row_blocks) > TQ_MAX_WG_LDS) waves /= 2;
            while (row_blocks > 1 && lds(waves, row_blocks) > TQ_MAX_WG_LDS) row_blocks /= 2;
            if (lds(waves, row_blocks) > TQ_MAX_WG_LDS)
                return tq_fail(TQ_ERR_UNSUPPORTED, "decode needs more LDS than a workgroup has");
        }
        for (int32_t i = 0; i < count; ++i) {
            const tq_prob_dev& P = probs[(size_t)i];
            const int64_t NB = (P.N + 63) / 64;
            for (int64_t rb = 0; rb < NB; rb += row_blocks) {
                const int64_t nb = std::min<int64_t>(row_blocks, NB - rb);
                items.push_back({nb * P.NC * (int64_t)K0, i, (int32_t)rb});
            }
        }
    }
    // longest items first, so that the last workgroups to start are short
    std::stable_sort(items.begin(), items.end(), [](const Item& a, const Item& b) { return a.cost > b.cost; });
    std::vector<uint8_t> host((size_t)need, 0);
    if (count > 0) memcpy(host.data(), probs.data(), (size_t)count * sizeof(tq_prob_dev));
    int32_t* it = (int32_t*)(host.data() + tq_ws_items_off(count));
    for (size_t j = 0; j < items.size(); ++j) {
        it[2 * j] = items[j].prob;
        it[2 * j + 1] = items[j].rb0;
    }
    hipStream_t st = (hipStream_t)stream;
    if ((s = tq_check_hip(hipMemcpyAsync(workspace, host.data(), need, hipMemcpyHostToDevice, st),
                          "tq_gemv_grouped_prepare copy")))
        return s;
    if ((s = tq_check_hip(hipStreamSynchronize(st), "tq_gemv_grouped_prepare synchronize"))) return s;
    plan->workspace = workspace;
    plan->n_items = (int64_t)items.size();
    plan->family = family;
    plan->x_type = x_type;
    plan->M = (int32_t)M;
    plan->waves = waves;
    plan->row_blocks = row_blocks;
    plan->n_problems = count;
    plan->x_lds_bytes = (int32_t)x_lds;
    plan->reserved = 0;
    return tq_ok();
}

TQ_EXPORT tq_status tq_gemv_grouped_run(const tq_grouped_plan* plan, void* stream)
{
    if (!plan) return tq_fail(TQ_ERR_ARG, "plan is NULL");
    if (plan->n_items == 0) return tq_ok();
    tq_status s;
    if ((s = tq_check_ptr(plan->workspace, "plan workspace", false))) return s;
    if (plan->n_items < 0 || plan->n_items > (1ll << 31) - 1 || plan->n_problems < 1)
        return tq_fail(TQ_ERR_ARG, "plan is not filled by tq_gemv_grouped_prepare");
    if (plan->family >= 1000) return tq_gemm_grouped_run(plan, stream);   // matrix-core plan
    if (plan->x_lds_bytes < 0 || plan->x_lds_bytes > TQ_MAX_Q8_LDS)
        return tq_fail(TQ_ERR_ARG, "plan is not filled by tq_gemv_grouped_prepare");
    if ((s = tq_gemv_launch_grouped(plan->family, plan->waves, plan->row_blocks, plan->workspace,
                                    plan->n_problems, plan->n_items, plan->x_lds_bytes,
                                    (hipStream_t)stream)))
        return s;
    return tq_ok();
}
