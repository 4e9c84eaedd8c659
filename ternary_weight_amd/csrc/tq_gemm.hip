// libtq: tq_gemm and tq_gemm_grouped_* -- prefill product on the matrix
// cores (validation and dispatch; the kernels are in tq_gemm_impl.h).
#include <string.h>

#include <algorithm>
#include <vector>

#include "tq_gemm_kernels.h"

namespace {

constexpr int64_t kMaxM = 1 << 24;
// int8 with one plane and a per-tensor scale and at least this many tokens
// (up to 16) runs on the wide few-token kernels, two 64-row blocks per wave.
#ifndef TQ_I8_WIDE_MIN_M
#define TQ_I8_WIDE_MIN_M 8
#endif
constexpr int kFamilyBase = 1000;   // grouped plans of tq_gemm carry family >= this

int gemm_row(const tq_layout& L, int x_type)
{
    if (L.layout == TQ_SCALE_TENSOR) return TQ_GEMM_ROW_TENSOR;
    if (L.layout == TQ_SCALE_CODEBOOK) return TQ_GEMM_ROW_CODEBOOK;
    if (L.layout == TQ_SCALE_CODEBOOK_B3) return TQ_GEMM_ROW_CODEBOOK_B3;
    if (x_type == TQ_BF16 && L.g % 32 != 0) return TQ_GEMM_ROW_GROUP16;
    return TQ_GEMM_ROW_GROUP;
}

// Kernel tables: 0 int8, 1 bf16, 2 bf16 with at most 16 tokens, 3 int8 with
// at most 16 tokens, 4 int8 with TQ_I8_WIDE_MIN_M to 16 tokens.
constexpr int kTables = 5;
int table_index(int x_type, int64_t M)
{
    const bool few = M <= TQ_MAX_M_GEMV;
    if (x_type == TQ_I8) return few ? (M >= TQ_I8_WIDE_MIN_M ? 4 : 3) : 0;
    return few ? 2 : 1;
}

const tq_gemm_kernel (*gemm_table(int index))[4]
{
    switch (index) {
    case 0: return tq_gemm_table_i8();
    case 1: return tq_gemm_table_bf16();
    case 2: return tq_gemm_table_bf16_skinny();
    case 3: return tq_gemm_table_i8_skinny();
    default: return tq_gemm_table_i8_skinny_wide();
    }
}

// Kernel for (x_type, layout, K, g, M), or null with the reason recorded.
const tq_gemm_kernel* gemm_kernel(const tq_layout& L, int x_type, int64_t M)
{
    if (x_type != TQ_I8 && x_type != TQ_BF16) {
        tq_fail(TQ_ERR_UNSUPPORTED, "tq_gemm takes TQ_I8 or TQ_BF16 activations (got %d)", x_type);
        return nullptr;
    }
    const tq_gemm_kernel* k = &gemm_table(table_index(x_type, M))[gemm_row(L, x_type)][L.K - 1];
    if (!k->single || (L.layout != TQ_SCALE_TENSOR && L.g % k->step != 0)) {
        tq_fail(TQ_ERR_UNSUPPORTED, "tq_gemm: no matrix-core kernel for this scale layout and group size %d "
                "with x_type %d (int8 steps are 64 columns)", L.g, x_type);
        return nullptr;
    }
    // the kernels address x, the codes and the scales with 32-bit offsets,
    // including the rows a partial tile reads past M and N
    const int64_t lim = (int64_t)UINT32_MAX;
    const int64_t xb = (M + 16 * k->fm * k->wm) * L.Kin * (x_type == TQ_I8 ? 1 : 2);
    const int64_t cb = (L.NB + 4 * k->fn) * L.NC * (L.layout == TQ_SCALE_CODEBOOK_B3 ? TQ_B3_CHUNK_BYTES : L.K * 1024);
    const int64_t sb = (L.NB + 4 * k->fn) * (tq_is_codebook(L.layout) ? L.NID : L.NGD * L.K) * 256;
    if (xb > lim || cb > lim || sb > lim) {
        tq_fail(TQ_ERR_UNSUPPORTED, "tq_gemm: an operand exceeds 4 GiB (x %lld, codes %lld bytes)", (long long)xb,
                (long long)cb);
        return nullptr;
    }
    return k;
}

int gemm_family(const tq_layout& L, int x_type, int64_t M)
{
    return kFamilyBase + (table_index(x_type, M) * TQ_GEMM_ROWS + gemm_row(L, x_type)) * 4 + L.K - 1;
}

const tq_gemm_kernel* kernel_of_family(int family)
{
    const int f = family - kFamilyBase;
    if (f < 0 || f >= kTables * TQ_GEMM_ROWS * 4) return nullptr;
    const tq_gemm_kernel* k = &gemm_table(f / (TQ_GEMM_ROWS * 4))[(f / 4) % TQ_GEMM_ROWS][f % 4];
    return k->single ? k : nullptr;
}

int64_t tiles_of(const tq_gemm_kernel& k, int64_t M, int64_t N, int64_t* tiles_m)
{
    const int64_t rows_m = 16 * k.fm * k.wm, rows_n = 16 * k.fn * (4 / k.wm);
    const int64_t tm = (M + rows_m - 1) / rows_m;
    const int64_t tn = (N + rows_n - 1) / rows_n;
    if (tiles_m) *tiles_m = tm;
    return tm * tn;
}

}  // namespace

bool tq_gemm_supports(const tq_layout& L, int x_type, int64_t M) { return gemm_kernel(L, x_type, M) != nullptr; }

tq_status tq_gemm_launch(const tq_layout& L, const tq_prob_dev& P, int x_type, hipStream_t stream)
{
    const tq_gemm_kernel* k = gemm_kernel(L, x_type, P.M);
    if (!k) return TQ_ERR_UNSUPPORTED;
    int64_t tiles_m = 0;
    const int64_t tiles = tiles_of(*k, P.M, L.N, &tiles_m);
    if (tiles > INT32_MAX) return tq_fail(TQ_ERR_UNSUPPORTED, "tq_gemm: %lld tiles exceed one launch", (long long)tiles);
    hipLaunchKernelGGL(k->single, dim3((unsigned)tiles), dim3(256), 0, stream, P, (int)tiles_m);
    return tq_check_launch("tq_gemm");
}

TQ_EXPORT tq_status tq_gemm(const tq_weight_desc* desc, const void* blob, int64_t M, int32_t x_type,
                            const void* x, const float* x_scale, float* y, int32_t* acc, void* stream)
{
    tq_layout L;
    tq_status s = tq_check_desc(desc, &L);
    if (s) return s;
    if ((s = tq_check_call(L, blob, M, x_type, x, x_scale, y, acc, kMaxM, 16))) return s;
    if (!gemm_kernel(L, x_type, M)) return TQ_ERR_UNSUPPORTED;
    if (M == 0 || L.N == 0) return tq_ok();
    const tq_prob_dev P = tq_make_prob(L, blob, M, x, x_scale, y, acc);
    if ((s = tq_gemm_launch(L, P, x_type, (hipStream_t)stream))) return s;
    return tq_ok();
}

TQ_EXPORT tq_status tq_gemm_grouped_workspace_size(const tq_problem* problems, int32_t count, int64_t M,
                                                   int32_t x_type, size_t* bytes)
{
    if (!bytes) return tq_fail(TQ_ERR_ARG, "bytes is NULL");
    if (count < 0 || (count > 0 && !problems)) return tq_fail(TQ_ERR_ARG, "bad problem list");
    if (M < 0 || M > kMaxM) return tq_fail(TQ_ERR_UNSUPPORTED, "M = %lld not in 0..%lld", (long long)M,
                                           (long long)kMaxM);
    int64_t items = 0;
    for (int32_t i = 0; i < count; ++i) {
        tq_layout L;
        tq_status s = tq_check_desc(problems[i].desc, &L);
        if (s) return tq_fail_problem(s, i);
        const tq_gemm_kernel* k = gemm_kernel(L, x_type, M);
        if (!k) return tq_fail_problem(TQ_ERR_UNSUPPORTED, i);
        items += tiles_of(*k, M, L.N, nullptr);
    }
    if (items > INT32_MAX) return tq_fail(TQ_ERR_UNSUPPORTED, "%lld tiles exceed one launch", (long long)items);
    *bytes = (size_t)(tq_ws_items_off(count) + tq_align256(items * 8));
    if (*bytes == 0) *bytes = 256;
    return tq_ok();
}

// tokens (host, may be NULL): problem i's own token count, at most M; the
// kernel is the one of M tokens, each problem's tiles cover its own count.
tq_status tq_gemm_grouped_prepare_counts(const tq_problem* problems, const int32_t* tokens, int32_t count,
                                         int64_t M, int32_t x_type, void* workspace, size_t workspace_bytes,
                                         tq_grouped_plan* plan, void* stream)
{
    if (!plan) return tq_fail(TQ_ERR_ARG, "plan is NULL");
    size_t need = 0;
    tq_status s = tq_gemm_grouped_workspace_size(problems, count, M, x_type, &need);
    if (s) return s;
    if ((s = tq_check_ptr(workspace, "workspace", false))) return s;
    if (workspace_bytes < need)
        return tq_fail(TQ_ERR_ARG, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    std::vector<tq_prob_dev> probs((size_t)count);
    struct Item { int64_t cost; int32_t prob, tile; };
    std::vector<Item> items;
    int family = -1;
    const tq_gemm_kernel* k0 = nullptr;
    for (int32_t i = 0; i < count; ++i) {
        const tq_problem& pr = problems[i];
        tq_layout L;
        tq_check_desc(pr.desc, &L);
        const int64_t Mi = tokens ? tokens[i] : M;
        if (Mi < 0 || Mi > M)
            return tq_fail(TQ_ERR_ARG, "problem %d: %lld tokens, not in 0..%lld", i, (long long)Mi, (long long)M);
        if ((s = tq_check_call(L, pr.blob, Mi, x_type, pr.x, pr.x_scale, pr.y, pr.acc, kMaxM, 16)))
            return tq_fail_problem(s, i);
        const tq_gemm_kernel* k = gemm_kernel(L, x_type, M);
        if (i == 0) {
            family = gemm_family(L, x_type, M);
            k0 = k;
        } else if (gemm_family(L, x_type, M) != family) {
            return tq_fail(TQ_ERR_UNSUPPORTED,
                           "problem %d: all problems of a plan must share planes, layout and x_type", i);
        }
        probs[(size_t)i] = tq_make_prob(L, pr.blob, Mi, pr.x, pr.x_scale, pr.y, pr.acc);
        if (Mi > 0) {
            const int64_t n = tiles_of(*k, Mi, L.N, nullptr);
            for (int64_t t = 0; t < n; ++t) items.push_back({L.Kin * (int64_t)L.K, i, (int32_t)t});
        }
    }
    // longest problems first, so that the last workgroups to start are short
    std::stable_sort(items.begin(), items.end(), [](const Item& a, const Item& b) { return a.cost > b.cost; });
    std::vector<uint8_t> host(need, 0);
    if (count > 0) memcpy(host.data(), probs.data(), (size_t)count * sizeof(tq_prob_dev));
    int32_t* it = (int32_t*)(host.data() + tq_ws_items_off(count));
    for (size_t j = 0; j < items.size(); ++j) {
        it[2 * j] = items[j].prob;
        it[2 * j + 1] = items[j].tile;
    }
    hipStream_t st = (hipStream_t)stream;
    if ((s = tq_check_hip(hipMemcpyAsync(workspace, host.data(), need, hipMemcpyHostToDevice, st),
                          "tq_gemm_grouped_prepare copy")))
        return s;
    if ((s = tq_check_hip(hipStreamSynchronize(st), "tq_gemm_grouped_prepare synchronize"))) return s;
    memset(plan, 0, sizeof *plan);
    plan->workspace = workspace;
    plan->n_items = (int64_t)items.size();
    plan->family = family;
    plan->x_type = x_type;
    plan->M = (int32_t)M;
    plan->waves = 4;
    plan->row_blocks = k0 ? k0->fn * (4 / k0->wm) / 4 : 0;
    plan->n_problems = count;
    return tq_ok();
}

TQ_EXPORT tq_status tq_gemm_grouped_prepare(const tq_problem* problems, int32_t count, int64_t M,
                                            int32_t x_type, void* workspace, size_t workspace_bytes,
                                            tq_grouped_plan* plan, void* stream)
{
    return tq_gemm_grouped_prepare_counts(problems, nullptr, count, M, x_type, workspace, workspace_bytes, plan,
                                          stream);
}

TQ_EXPORT tq_status tq_gemm_grouped_run(const tq_grouped_plan* plan, void* stream)
{
    if (!plan) return tq_fail(TQ_ERR_ARG, "plan is NULL");
    if (plan->n_items == 0) return tq_ok();
    tq_status s;
    if ((s = tq_check_ptr(plan->workspace, "plan workspace", false))) return s;
    const tq_gemm_kernel* k = kernel_of_family(plan->family);
    if (!k || plan->n_items < 0 || plan->n_items > INT32_MAX || plan->n_problems < 1)
        return tq_fail(TQ_ERR_ARG, "plan is not filled by tq_gemm_grouped_prepare");
    const uint8_t* ws = (const uint8_t*)plan->workspace;
    hipLaunchKernelGGL(k->grouped, dim3((unsigned)plan->n_items), dim3(256), 0, (hipStream_t)stream,
                       (const tq_prob_dev*)ws, (const int2*)(ws + tq_ws_items_off(plan->n_problems)));
    if ((s = tq_check_launch("tq_gemm_grouped_run"))) return s;
    return tq_ok();
}
