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
    P.cb = tq_is_codebook(L.layout) ? (const uint16_t*)(b + L.cb_off) : nullptr;
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
    if (tq_gemv_uses_mfma(x_type, L.layout, M, x) && tq_gemm_supports(L, x_type, M))
        s = tq_gemm_launch(L, P, x_type, (hipStream_t)stream);
    else
        s = tq_gemv_launch_single(L, P, x_type, (hipStream_t)stream);
    if (s) return s;
    return tq_ok();
}

// Waves per workgroup of a bf16 plan with an item per wave (they share the
// 64 KiB trit table).
#ifndef TQ_BF16_WAVE_WG
#define TQ_BF16_WAVE_WG 16
#endif

namespace {

int64_t pass_slices(int64_t M) { return M <= TQ_PASS_TOKENS ? 1 : (M + TQ_PASS_TOKENS - 1) / TQ_PASS_TOKENS; }

}  // namespace

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
    // a problem of more than one pass of tokens is cut into slices, each an
    // entry of the table with its own items, placed with holes between
    const int64_t slices = pass_slices(M);
    // with per-wave items a row block's slices never straddle workgroups,
    // which leaves fewer holes than items, plus the last workgroup's
    if (slices > 1) items = 2 * items * slices + 8 * (slices + 1) + 16;
    // problem entries, then one (entry, first row block) item per workgroup
    *bytes = (size_t)(tq_ws_items_off(count * slices) + tq_align256(items * 8));
    if (*bytes == 0) *bytes = 256;
    return tq_ok();
}

namespace {

// The decode plan; tokens (host, may be NULL): each problem's own token
// count, every one at most M.  The kernels take TQ_PASS_TOKENS tokens per
// pass over the codes; a problem with more is cut into slices of that many
// tokens, each an entry of the device table.  The slices of one
// row block are placed 8 workgroup items apart (workgroups are dealt to the
// 8 XCDs in turn, so they run on one XCD at about the same time), or, for
// bf16, in consecutive waves of one workgroup (an item per wave).  Holes
// left by either placement are items of entry -1.
tq_status grouped_prepare(const tq_problem* problems, const int32_t* tokens, int32_t count, int64_t M,
                          int32_t x_type, void* workspace, size_t workspace_bytes, tq_grouped_plan* plan,
                          void* stream)
{
    if (!plan) return tq_fail(TQ_ERR_ARG, "plan is NULL");
    const int pow2[] = {1, 2, 4, 8, 16};
    auto is_shape = [&](int v) { for (int p : pow2) if (v == p) return true; return false; };
    int waves = plan->waves, row_blocks = plan->row_blocks;
    const bool hinted = is_shape(waves) && is_shape(row_blocks) && waves * row_blocks <= 16;
    size_t need = 0;
    tq_status s = tq_gemv_grouped_workspace_size(problems, count, M, &need);   // validates the descs
    if (s) return s;
    if (!hinted) {
        // bf16: the trit table fills 64 KiB of LDS, so 16 waves share it: 16
        // one-wave row blocks for one token, 4 two-wave row blocks for
        // several.  int8 over several tokens: 2 x 2 for one plane and a
        // per-tensor scale, one wave per row block otherwise.  Each was
        // measured ahead of the other shapes.
        const bool k1 = count > 0 && problems[0].desc->planes == 1 &&
                        problems[0].desc->scale_layout == TQ_SCALE_TENSOR;
        if (x_type == TQ_BF16) {
            waves = M > 1 ? 2 : 1;
            row_blocks = M > 1 ? 4 : 16;
        } else if (x_type == TQ_I8 && M > 1) {
            waves = k1 ? 2 : 1;
            row_blocks = k1 ? 2 : 4;
        } else {
            waves = x_type == TQ_F32_Q8 ? 1 : 4;
            row_blocks = x_type == TQ_F32_Q8 ? 4 : 1;
        }
    }
    // several bf16 or int8 tokens: the matrix-core kernels, if every x allows
    // 16-byte loads and no shape hint asks for the vector ALUs.  With
    // per-problem counts the measure is the mean count of the problems that
    // have tokens (a 16-token tile costs the same for 1 or 16; the vector
    // ALUs pay per pass of 4 tokens).
    int64_t busy = 0, sum = 0;
    for (int32_t i = 0; tokens && i < count; ++i) {
        busy += tokens[i] > 0;
        sum += std::max(tokens[i], 0);
    }
    const int64_t mfma_min = count > 0 ? tq_mfma_min_m(x_type, problems[0].desc->scale_layout) : INT64_MAX;
    bool mfma = count > 0 && !hinted && (x_type == TQ_BF16 || x_type == TQ_I8) &&
                (tokens ? sum >= mfma_min * std::max<int64_t>(busy, 1) : M >= mfma_min);
    for (int32_t i = 0; i < count && mfma; ++i) {
        mfma = ((uintptr_t)problems[i].x & 15) == 0;
        // a shape the matrix-core kernels do not take sends the plan to the vector ALUs
        tq_layout Li;
        if (mfma && problems[i].desc && tq_check_desc(problems[i].desc, &Li) == TQ_OK)
            mfma = tq_gemm_supports(Li, x_type, tokens ? std::max(tokens[i], 0) : M);
    }
    if (mfma)
        return tq_gemm_grouped_prepare_counts(problems, tokens, count, M, x_type, workspace, workspace_bytes, plan,
                                              stream);
    if ((s = tq_check_ptr(workspace, "workspace", false))) return s;
    if (workspace_bytes < need)
        return tq_fail(TQ_ERR_ARG, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    const int pass = TQ_PASS_TOKENS;
    std::vector<tq_prob_dev> probs;
    probs.reserve((size_t)count);
    struct Unit { int64_t cost; int32_t entry, n, rb0; };   // row blocks of one problem, all its slices
    std::vector<Unit> units;
    std::vector<int32_t> first((size_t)count), n_slices((size_t)count);
    int family = -1, K0 = 0, layout0 = -1, g0 = 0;
    size_t x_lds = 0;
    for (int32_t i = 0; i < count; ++i) {
        const tq_problem& pr = problems[i];
        tq_layout L;
        tq_check_desc(pr.desc, &L);
        const int64_t Mi = tokens ? tokens[i] : M;
        if (Mi < 0 || Mi > M)
            return tq_fail(TQ_ERR_ARG, "problem %d: %lld tokens, not in 0..%lld", i, (long long)Mi, (long long)M);
        if ((s = tq_check_call(L, pr.blob, Mi, x_type, pr.x, pr.x_scale, pr.y, pr.acc, TQ_MAX_M_GEMV)))
            return tq_fail_problem(s, i);
        if (i == 0) {
            K0 = L.K;
            layout0 = L.layout;
            g0 = L.g;
        } else if (L.K != K0 || L.layout != layout0 || (L.layout != TQ_SCALE_TENSOR && L.g != g0)) {
            return tq_fail(TQ_ERR_UNSUPPORTED,
                           "problem %d: all problems of a plan must share planes, layout and group", i);
        }
        const tq_prob_dev whole = tq_make_prob(L, pr.blob, Mi, pr.x, pr.x_scale, pr.y, pr.acc);
        first[(size_t)i] = (int32_t)probs.size();
        if (Mi <= pass) {
            probs.push_back(whole);
        } else {
            for (int m0 = 0; m0 < (int)Mi; m0 += pass)
                probs.push_back(tq_prob_slice(whole, x_type, m0, std::min<int>(pass, (int)Mi - m0)));
        }
        n_slices[(size_t)i] = (int32_t)probs.size() - first[(size_t)i];
        if (x_type == TQ_F32_Q8) x_lds = std::max(x_lds, tq_x_lds_bytes(std::min<int64_t>(Mi, pass), L.Kin));
    }
    bool sliced = false;
    for (int32_t i = 0; i < count; ++i) sliced = sliced || n_slices[(size_t)i] > 1;
    // bf16: per-wave items, the slices of a row block in one workgroup whose
    // 16 waves share the trit table (measured ahead of workgroup items of 16
    // row blocks; with int8 activations the two measured alike)
    const bool wave_mode = sliced && !hinted && x_type == TQ_BF16 && !tq_is_codebook(layout0);
    const int wave_wg = TQ_BF16_WAVE_WG;
    if (count > 0 && M > 0) {
        family = tq_gemv_family(x_type, layout0, K0, (int)std::min<int64_t>(M, pass));
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
        const int unit_blocks = wave_mode ? 1 : row_blocks;
        for (int32_t i = 0; i < count; ++i) {
            const tq_prob_dev& P = probs[(size_t)first[(size_t)i]];
            if (P.M == 0) continue;          // a problem with no tokens has no work
            const int64_t NB = (P.N + 63) / 64;
            for (int64_t rb = 0; rb < NB; rb += unit_blocks) {
                const int64_t nb = std::min<int64_t>(unit_blocks, NB - rb);
                units.push_back({nb * P.NC * (int64_t)K0, first[(size_t)i], n_slices[(size_t)i], (int32_t)rb});
            }
        }
    }
    // longest units first, so that the last workgroups to start are short
    std::stable_sort(units.begin(), units.end(), [](const Unit& a, const Unit& b) { return a.cost > b.cost; });
    std::vector<int2> items;
    if (wave_mode) {
        // a row block's slices (at most 4) in consecutive waves of one workgroup
        for (const Unit& u : units) {
            const int free = wave_wg - (int)(items.size() % wave_wg);
            if (u.n > free) items.resize(items.size() + free, make_int2(-1, 0));
            for (int j = 0; j < u.n; ++j) items.push_back(make_int2(u.entry + j, u.rb0));
        }
        items.resize((items.size() + wave_wg - 1) / wave_wg * wave_wg, make_int2(-1, 0));
        waves = 1;
        row_blocks = wave_wg;
    } else if (!sliced) {
        for (const Unit& u : units) items.push_back(make_int2(u.entry, u.rb0));
    } else {
        // each unit goes to the XCD whose list is shortest, its slices 8 items apart
        int64_t next[8];
        for (int r = 0; r < 8; ++r) next[r] = r;
        for (const Unit& u : units) {
            const int r = (int)(std::min_element(next, next + 8) - next);
            for (int j = 0; j < u.n; ++j) {
                const size_t pos = (size_t)(next[r] + 8 * j);
                if (items.size() <= pos) items.resize(pos + 1, make_int2(-1, 0));
                items[pos] = make_int2(u.entry + j, u.rb0);
            }
            next[r] += 8 * (int64_t)u.n;
        }
    }
    const int64_t n_entries = (int64_t)probs.size();
    if ((size_t)(tq_ws_items_off(n_entries) + (int64_t)items.size() * 8) > need)
        return tq_fail(TQ_ERR_ARG, "internal: plan exceeds its workspace");
    std::vector<uint8_t> host((size_t)need, 0);
    if (n_entries > 0) memcpy(host.data(), probs.data(), (size_t)n_entries * sizeof(tq_prob_dev));
    if (!items.empty())
        memcpy(host.data() + tq_ws_items_off(n_entries), items.data(), items.size() * sizeof(int2));
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
    plan->n_problems = (int32_t)n_entries;
    plan->x_lds_bytes = (int32_t)x_lds;
    plan->mode = wave_mode ? 1 : 0;
    return tq_ok();
}

}  // namespace

TQ_EXPORT tq_status tq_gemv_grouped_prepare(const tq_problem* problems, int32_t count, int64_t M,
                                            int32_t x_type, void* workspace, size_t workspace_bytes,
                                            tq_grouped_plan* plan, void* stream)
{
    return grouped_prepare(problems, nullptr, count, M, x_type, workspace, workspace_bytes, plan, stream);
}

TQ_EXPORT tq_status tq_gemv_grouped_prepare_tokens(const tq_problem* problems, const int32_t* tokens,
                                                   int32_t count, int32_t x_type, void* workspace,
                                                   size_t workspace_bytes, tq_grouped_plan* plan, void* stream)
{
    if (count > 0 && !tokens) return tq_fail(TQ_ERR_ARG, "tokens is NULL");
    int64_t M = 0;
    for (int32_t i = 0; i < count; ++i) M = std::max<int64_t>(M, tokens[i]);
    if (M > TQ_MAX_M_GEMV)
        return tq_fail(TQ_ERR_UNSUPPORTED, "a problem has more than %d tokens", TQ_MAX_M_GEMV);
    return grouped_prepare(problems, tokens, count, M, x_type, workspace, workspace_bytes, plan, stream);
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
    if (plan->mode == 1)
        return tq_gemv_launch_wave_items(plan->family, plan->row_blocks, plan->workspace, plan->n_problems,
                                         plan->n_items, (hipStream_t)stream);
    if (plan->mode != 0) return tq_fail(TQ_ERR_ARG, "plan is not filled by tq_gemv_grouped_prepare");
    if (plan->x_lds_bytes < 0 || plan->x_lds_bytes > TQ_MAX_Q8_LDS)
        return tq_fail(TQ_ERR_ARG, "plan is not filled by tq_gemv_grouped_prepare");
    if ((s = tq_gemv_launch_grouped(plan->family, plan->waves, plan->row_blocks, plan->workspace,
                                    plan->n_problems, plan->n_items, plan->x_lds_bytes,
                                    (hipStream_t)stream)))
        return s;
    return tq_ok();
}
