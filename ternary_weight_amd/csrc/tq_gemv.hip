// libtq: decode dispatch -- picks the kernel family and the workgroup shape.
#include "tq_gemv_impl.h"

namespace {

using namespace tqk;

int mt_index(int M) { return M <= 1 ? 0 : 1; }

// LDS of the partial sums: one area per wave when a row block is split.
size_t red_bytes(int family, int split_waves, int total_waves)
{
    if (split_waves <= 1) return 0;
    const int mti = family % kTiers, K = (family / kTiers) % 4 + 1, layout = (family / (4 * kTiers)) % kLayouts;
    const int R = layout != TQ_SCALE_TENSOR ? kMT[mti] : kMT[mti] * K;
    return (size_t)total_waves * R * 64 * 4;
}

const single_fn* single_tab(int xt, int mti)
{
    static const single_fn* (*const f[kXTypes][kTiers])() = {
        {single_table_0_0, single_table_0_1},
        {single_table_1_0, single_table_1_1},
        {single_table_2_0, single_table_2_1},
        {single_table_3_0, single_table_3_1}};
    return f[xt][mti]();
}

const grouped_fn* grouped_tab(int xt, int mti)
{
    static const grouped_fn* (*const f[kXTypes][kTiers])() = {
        {grouped_table_0_0, grouped_table_0_1},
        {grouped_table_1_0, grouped_table_1_1},
        {grouped_table_2_0, grouped_table_2_1},
        {grouped_table_3_0, grouped_table_3_1}};
    return f[xt][mti]();
}

// family = ((x_type * kLayouts + layout) * 4 + (K - 1)) * kTiers + M tier
constexpr int kPerTable = 4 * kLayouts;

single_fn single_of(int family)
{
    const int mti = family % kTiers, rest = family / kTiers;
    const single_fn* t = single_tab(rest / kPerTable, mti);
    return t ? t[rest % kPerTable] : nullptr;
}

grouped_fn grouped_of(int family)
{
    const int mti = family % kTiers, rest = family / kTiers;
    const grouped_fn* t = grouped_tab(rest / kPerTable, mti);
    return t ? t[rest % kPerTable] : nullptr;
}

wave_items_fn wave_items_fn_of(int family)
{
    const int mti = family % kTiers, rest = family / kTiers, xt = rest / kPerTable;
    if (mti != 1 || xt != TQ_BF16) return nullptr;
    return wave_table_1_1()[rest % kPerTable];
}

}  // namespace

size_t tq_gemv_lds_bytes(int family, int split_waves, int total_waves, size_t x_lds_bytes)
{
    const int x_type = family / kPerXT, layout = (family / (4 * kTiers)) % kLayouts, mti = family % kTiers;
    const size_t lut = layout == TQ_SCALE_CODEBOOK_B3 ? (size_t)(mti == 0 ? B3Table<16>::kBytes : B3Table<8>::kBytes)
                                                      : (size_t)kLutBytes;
    const size_t fixed = (x_type == TQ_BF16 ? lut : 0) + 1024;
    return fixed + red_bytes(family, split_waves, total_waves) + x_lds_bytes;
}

int tq_gemv_family(int x_type, int layout, int K, int M)
{
    if (x_type < 0 || x_type >= kXTypes || layout < 0 || layout >= kLayouts || K < 1 || K > 4 || M < 1 ||
        M > TQ_PASS_TOKENS)
        return -1;
    if (layout == TQ_SCALE_CODEBOOK_B3) {
        // the three digits decode to one combined value: kernel K = 1, bf16 only
        if (x_type != TQ_BF16 || K != 3) return -1;
        K = 1;
    }
    return ((x_type * kLayouts + layout) * 4 + (K - 1)) * kTiers + mt_index(M);
}

namespace {

tq_status launch_single(const tq_layout& L, const tq_prob_dev& P, int x_type, hipStream_t stream)
{
    const int fam = tq_gemv_family(x_type, L.layout, L.K, P.M);
    if (fam < 0) return tq_fail(TQ_ERR_UNSUPPORTED, "no decode kernel for this combination");
    // enough waves to cover the chip: split the columns of each row block
    const int cpu = (L.layout == TQ_SCALE_TENSOR || L.g <= 64) ? 1 : L.g / 64;
    const int64_t nunits = (L.NC + cpu - 1) / cpu;
    int waves = 1;
    const int64_t target = 4 * (int64_t)tq_device_cus();
    while (waves < 16 && L.NB * waves < target && nunits >= 4 * waves * 2) waves *= 2;
    if (x_type == TQ_BF16) waves = 16;   // the 64 KiB trit table is shared by up to 16 waves
    const size_t x_lds = x_type == TQ_F32_Q8 ? tq_x_lds_bytes(P.M, L.Kin) : 0;
    while (waves > 1 && tq_gemv_lds_bytes(fam, waves, waves, x_lds) > TQ_MAX_WG_LDS) waves /= 2;
    if (tq_gemv_lds_bytes(fam, waves, waves, x_lds) > TQ_MAX_WG_LDS)
        return tq_fail(TQ_ERR_UNSUPPORTED, "decode needs more LDS than a workgroup has");
    const size_t lds = red_bytes(fam, waves, waves) + x_lds;
    const single_fn fn = single_of(fam);
    if (!fn) return tq_fail(TQ_ERR_UNSUPPORTED, "no decode kernel for this combination");
    hipLaunchKernelGGL(fn, dim3((unsigned)L.NB), dim3(64 * waves), lds, stream, P);
    return tq_check_launch("tq_gemv");
}

}  // namespace

// More tokens than one pass takes: one launch per slice of tokens (the
// codes of the later launches come from the caches when the weight fits).
tq_status tq_gemv_launch_single(const tq_layout& L, const tq_prob_dev& P, int x_type, hipStream_t stream)
{
    for (int m0 = 0; m0 < P.M; m0 += TQ_PASS_TOKENS) {
        const tq_status s =
            launch_single(L, tq_prob_slice(P, x_type, m0, std::min(TQ_PASS_TOKENS, P.M - m0)), x_type, stream);
        if (s) return s;
    }
    return TQ_OK;
}

tq_status tq_gemv_launch_grouped(int family, int waves, int row_blocks, const void* workspace,
                                 int64_t n_probs, int64_t n_items, int x_lds_bytes, hipStream_t stream)
{
    if (family < 0 || family >= kPerXT * kXTypes) return tq_fail(TQ_ERR_ARG, "bad plan family %d", family);
    if (waves < 1 || row_blocks < 1 || waves * row_blocks > 16)
        return tq_fail(TQ_ERR_ARG, "bad plan shape %d x %d", waves, row_blocks);
    const grouped_fn fn = grouped_of(family);
    if (!fn) return tq_fail(TQ_ERR_ARG, "bad plan family %d", family);
    if (n_items <= 0) return tq_ok();
    const uint8_t* ws = (const uint8_t*)workspace;
    const tq_prob_dev* probs = (const tq_prob_dev*)ws;
    const int2* items = (const int2*)(ws + tq_ws_items_off(n_probs));
    const int total = waves * row_blocks;
    if (tq_gemv_lds_bytes(family, waves, total, (size_t)x_lds_bytes) > TQ_MAX_WG_LDS)
        return tq_fail(TQ_ERR_UNSUPPORTED, "plan shape %d x %d needs more LDS than a workgroup has", waves,
                       row_blocks);
    const size_t lds = red_bytes(family, waves, total) + (size_t)x_lds_bytes;
    hipLaunchKernelGGL(fn, dim3((unsigned)n_items), dim3(64 * total), lds, stream, probs, items, row_blocks);
    return tq_check_launch("tq_gemv_grouped_run");
}

tq_status tq_gemv_launch_wave_items(int family, int waves, const void* workspace, int64_t n_probs,
                                    int64_t wave_items, hipStream_t stream)
{
    if (family < 0 || family >= kPerXT * kXTypes) return tq_fail(TQ_ERR_ARG, "bad plan family %d", family);
    if (waves < 1 || waves > 16 || wave_items % waves != 0)
        return tq_fail(TQ_ERR_ARG, "bad per-wave plan: %lld items, %d waves", (long long)wave_items, waves);
    const wave_items_fn fn = wave_items_fn_of(family);
    if (!fn) return tq_fail(TQ_ERR_ARG, "no per-wave kernel for plan family %d", family);
    if (wave_items <= 0) return tq_ok();
    const uint8_t* ws = (const uint8_t*)workspace;
    const tq_prob_dev* probs = (const tq_prob_dev*)ws;
    const int2* items = (const int2*)(ws + tq_ws_items_off(n_probs));
    hipLaunchKernelGGL(fn, dim3((unsigned)(wave_items / waves)), dim3(64 * waves), 0, stream, probs, items);
    return tq_check_launch("tq_gemv_grouped_run");
}
