// libtq: status handling, descriptor validation and size accounting.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "tq_internal.h"

static thread_local char g_last_error[512];

tq_status tq_fail(tq_status s, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return s;
}

tq_status tq_ok()
{
    g_last_error[0] = 0;
    return TQ_OK;
}

TQ_EXPORT int32_t tq_abi_version(void) { return TQ_ABI_VERSION; }

TQ_EXPORT const char* tq_status_string(int32_t s)
{
    switch (s) {
    case TQ_OK: return "ok";
    case TQ_ERR_ARG: return "invalid argument";
    case TQ_ERR_SHAPE: return "invalid shape";
    case TQ_ERR_ALIGN: return "misaligned pointer";
    case TQ_ERR_VALUE: return "invalid value";
    case TQ_ERR_UNSUPPORTED: return "unsupported combination";
    case TQ_ERR_DEVICE: return "device error";
    default: return "unknown status";
    }
}

TQ_EXPORT const char* tq_last_error(void) { return g_last_error; }

static bool pow2_group(int g) { return g == 16 || g == 32 || g == 64 || g == 128 || g == 256; }

tq_status tq_check_desc(const tq_weight_desc* d, tq_layout* L)
{
    if (!d) return tq_fail(TQ_ERR_ARG, "desc is NULL");
    if (d->planes < 1 || d->planes > 4)
        return tq_fail(TQ_ERR_ARG, "planes = %d, must be 1..4", d->planes);
    if (d->scale_layout < TQ_SCALE_TENSOR || d->scale_layout > TQ_SCALE_CODEBOOK_B3)
        return tq_fail(TQ_ERR_ARG, "scale_layout = %d is not a tq_scale_layout", d->scale_layout);
    if (d->out_features < 0 || d->in_features < 0)
        return tq_fail(TQ_ERR_ARG, "negative shape %lld x %lld", (long long)d->out_features,
                       (long long)d->in_features);
    if (d->out_features > TQ_MAX_N || d->in_features > TQ_MAX_KIN)
        return tq_fail(TQ_ERR_SHAPE, "shape %lld x %lld exceeds %d x %d",
                       (long long)d->out_features, (long long)d->in_features, TQ_MAX_N, TQ_MAX_KIN);
    if (d->in_features % 16)
        return tq_fail(TQ_ERR_SHAPE, "in_features = %lld is not a multiple of 16",
                       (long long)d->in_features);
    if (d->scale_layout != TQ_SCALE_TENSOR) {
        if (!pow2_group(d->group))
            return tq_fail(TQ_ERR_ARG, "group = %d, must be 16, 32, 64, 128 or 256", d->group);
        if (d->in_features % d->group)
            return tq_fail(TQ_ERR_SHAPE, "in_features = %lld is not a multiple of group %d",
                           (long long)d->in_features, d->group);
    }
    if (tq_is_codebook(d->scale_layout) && (d->n_codebook < 1 || d->n_codebook > TQ_CB_SLOTS))
        return tq_fail(TQ_ERR_ARG, "n_codebook = %d, must be 1..%d", d->n_codebook, TQ_CB_SLOTS);
    if (d->scale_layout == TQ_SCALE_CODEBOOK_B3 && d->planes != 3)
        return tq_fail(TQ_ERR_UNSUPPORTED, "TQ_SCALE_CODEBOOK_B3 packs three digits per weight (planes = %d)",
                       d->planes);
    if (L) tq_layout_make(d, L);
    return TQ_OK;
}

tq_status tq_check_ptr(const void* p, const char* name, bool nullable, int align)
{
    if (!p) return nullable ? TQ_OK : tq_fail(TQ_ERR_ARG, "%s is NULL", name);
    if (((uintptr_t)p) & (uintptr_t)(align - 1))
        return tq_fail(TQ_ERR_ALIGN, "%s = %p is not %d-byte aligned", name, p, align);
    return TQ_OK;
}

tq_status tq_check_hip(hipError_t e, const char* what)
{
    if (e == hipSuccess) return TQ_OK;
    return tq_fail(TQ_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

tq_status tq_check_launch(const char* what) { return tq_check_hip(hipGetLastError(), what); }

int tq_device_cus()
{
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (!cache[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

TQ_EXPORT tq_status tq_packed_size(const tq_weight_desc* desc, size_t* bytes)
{
    tq_layout L;
    tq_status s = tq_check_desc(desc, &L);
    if (s) return s;
    if (!bytes) return tq_fail(TQ_ERR_ARG, "bytes is NULL");
    *bytes = (size_t)L.total;
    return tq_ok();
}
