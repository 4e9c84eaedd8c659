// libtq: tq_pack / tq_unpack -- canonical planes and scales <-> device blob.
//
// Packing follows the two-bit code of the QORA-LLM-2B page ("Ternary GEMV (No
// Multiplication)": four trits per byte, two bits each) with 00 = 0, 01 = +1,
// 10 = -1, in the lane-slot order documented in tq_layout.h.
#include "tq_internal.h"

namespace {

constexpr int kBlock = 256;

__global__ void k_write_header(tq_blob_header* h, tq_weight_desc d)
{
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        tq_blob_header v = {};
        v.magic = TQ_BLOB_MAGIC;
        v.version = TQ_BLOB_VERSION;
        v.planes = d.planes;
        v.group = d.scale_layout == TQ_SCALE_TENSOR ? 0 : d.group;
        v.scale_layout = d.scale_layout;
        v.n_codebook = tq_is_codebook(d.scale_layout) ? d.n_codebook : 0;
        v.out_features = d.out_features;
        v.in_features = d.in_features;
        v.pack_status = 0;
        *h = v;
    }
}

__device__ __forceinline__ uint32_t code_of(int8_t t) { return t == 1 ? 1u : (t == -1 ? 2u : 0u); }

// One thread per code dword (16 trits); dword index t is also its offset / 4.
__global__ void k_pack_codes(const int8_t* __restrict__ trits, uint32_t* __restrict__ codes,
                             uint32_t* status, int64_t total, int K, int64_t N, int64_t Kin,
                             int64_t NC)
{
    uint32_t bad = 0;
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int d = (int)(t & 3);
        const int lane = (int)((t >> 2) & 63);
        int64_t rest = t >> 8;
        const int k = (int)(rest % K);
        rest /= K;
        const int64_t c = rest % NC;
        const int64_t rb = rest / NC;
        const int64_t n = rb * TQ_ROWS + lane;
        const int64_t col0 = c * TQ_CHUNK + 16 * d;
        uint32_t w = 0;
        if (n < N && col0 < Kin) {
            const int4 v = *reinterpret_cast<const int4*>(trits + ((int64_t)k * N + n) * Kin + col0);
            const uint32_t b[4] = {(uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w};
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int8_t tv = (int8_t)((b[q >> 2] >> (8 * (q & 3))) & 0xFF);
                if (tv < -1 || tv > 1) bad |= TQ_PACK_BAD_TRIT;
                // column 4p + byte b -> byte b, bits 2p..2p+1
                const int p = q >> 2, byte = q & 3;
                w |= code_of(tv) << (8 * byte + 2 * p);
            }
        }
        codes[t] = w;
    }
    if (bad) atomicOr(status, bad);
}

__global__ void k_unpack_codes(const uint32_t* __restrict__ codes, int8_t* __restrict__ trits,
                               int64_t total, int K, int64_t N, int64_t Kin, int64_t NC)
{
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int d = (int)(t & 3);
        const int lane = (int)((t >> 2) & 63);
        int64_t rest = t >> 8;
        const int k = (int)(rest % K);
        rest /= K;
        const int64_t c = rest % NC;
        const int64_t rb = rest / NC;
        const int64_t n = rb * TQ_ROWS + lane;
        const int64_t col0 = c * TQ_CHUNK + 16 * d;
        if (n >= N || col0 >= Kin) continue;
        const uint32_t w = codes[t];
        uint32_t b[4] = {0, 0, 0, 0};
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int p = q >> 2, byte = q & 3;
            const uint32_t c2 = (w >> (8 * byte + 2 * p)) & 3u;
            const int tv = (int)(c2 & 1u) - (int)(c2 >> 1);     // 11 reads as 0
            b[q >> 2] |= ((uint32_t)(uint8_t)(int8_t)tv) << (8 * (q & 3));
        }
        *reinterpret_cast<int4*>(trits + ((int64_t)k * N + n) * Kin + col0) =
            make_int4((int)b[0], (int)b[1], (int)b[2], (int)b[3]);
    }
}

__device__ __forceinline__ bool f16_finite(uint16_t h) { return (h & 0x7C00u) != 0x7C00u; }

// GROUP_F16: one thread per scale dword (two groups).
__global__ void k_pack_group_scales(const uint16_t* __restrict__ s, uint32_t* __restrict__ out,
                                    uint32_t* status, int64_t total, int K, int64_t N, int64_t G,
                                    int64_t NGD, int unpack, uint16_t* __restrict__ s_out)
{
    uint32_t bad = 0;
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int lane = (int)(t & 63);
        int64_t rest = t >> 6;
        const int k = (int)(rest % K);
        rest /= K;
        const int64_t gd = rest % NGD;
        const int64_t rb = rest / NGD;
        const int64_t n = rb * TQ_ROWS + lane;
        if (!unpack) {
            uint32_t w = 0;
            for (int h = 0; h < 2; ++h) {
                const int64_t grp = 2 * gd + h;
                if (n < N && grp < G) {
                    const uint16_t v = s[((int64_t)k * N + n) * G + grp];
                    if (!f16_finite(v)) bad |= TQ_PACK_BAD_SCALE;
                    w |= (uint32_t)v << (16 * h);
                }
            }
            out[t] = w;
        } else {
            const uint32_t w = out[t];
            for (int h = 0; h < 2; ++h) {
                const int64_t grp = 2 * gd + h;
                if (n < N && grp < G) s_out[((int64_t)k * N + n) * G + grp] = (uint16_t)(w >> (16 * h));
            }
        }
    }
    if (bad) atomicOr(status, bad);
}

// CODEBOOK_B3: one thread per (row block, chunk, lane) -- the 64 columns of
// one row in one chunk, three digit planes -> 32 ten-bit pair codes (the
// 320-bit stream of tq_layout.h, in its three parts).
__global__ void k_pack_b3(const int8_t* __restrict__ trits, uint8_t* __restrict__ codes, uint32_t* status,
                          int64_t total, int64_t N, int64_t Kin, int64_t NC)
{
    uint32_t bad = 0;
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int lane = (int)(t & 63);
        const int64_t rest = t >> 6;
        const int64_t c = rest % NC, rb = rest / NC;
        const int64_t n = rb * TQ_ROWS + lane;
        uint32_t w[10] = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
        if (n < N) {
            for (int q = 0; q < 4; ++q) {            // 16 columns at a time (Kin is a multiple of 16)
                const int64_t col0 = c * TQ_CHUNK + 16 * q;
                if (col0 >= Kin) break;
                int v[16];
                for (int i = 0; i < 16; ++i) v[i] = 0;
                for (int k = 0; k < 3; ++k) {       // digit plane k weighs 3^(2-k)
                    const int4 d = *reinterpret_cast<const int4*>(trits + ((int64_t)k * N + n) * Kin + col0);
                    const uint32_t b[4] = {(uint32_t)d.x, (uint32_t)d.y, (uint32_t)d.z, (uint32_t)d.w};
                    for (int i = 0; i < 16; ++i) {
                        const int tv = (int8_t)((b[i >> 2] >> (8 * (i & 3))) & 0xFF);
                        if (tv < -1 || tv > 1) bad |= TQ_PACK_BAD_TRIT;
                        v[i] = 3 * v[i] + tv;
                    }
                }
                for (int i = 0; i < 8; ++i) {       // pair j = 8q + i: columns 2j, 2j + 1
                    const uint32_t a = (uint32_t)((v[2 * i] % 27 + 27) % 27);
                    const uint32_t b = (uint32_t)((v[2 * i + 1] % 27 + 27) % 27);
                    const uint32_t code = (a + 27u * b) & 0x3FFu;
                    const int bit = 10 * (8 * q + i), dw = bit >> 5, sh = bit & 31;
                    w[dw] |= code << sh;
                    if (sh > 22) w[dw + 1] |= code >> (32 - sh);
                }
            }
        }
        uint8_t* blk = codes + (rb * NC + c) * TQ_B3_CHUNK_BYTES;
        *reinterpret_cast<uint4*>(blk + lane * 16) = make_uint4(w[0], w[1], w[2], w[3]);
        *reinterpret_cast<uint4*>(blk + 1024 + lane * 16) = make_uint4(w[4], w[5], w[6], w[7]);
        *reinterpret_cast<uint2*>(blk + 2048 + lane * 8) = make_uint2(w[8], w[9]);
    }
    if (bad) atomicOr(status, bad);
}

// Inverse of k_pack_b3: pair codes -> the three digit planes (codes >= 729,
// never written, read as zero weights).
__global__ void k_unpack_b3(const uint8_t* __restrict__ codes, int8_t* __restrict__ trits, int64_t total, int64_t N,
                            int64_t Kin, int64_t NC)
{
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int lane = (int)(t & 63);
        const int64_t rest = t >> 6;
        const int64_t c = rest % NC, rb = rest / NC;
        const int64_t n = rb * TQ_ROWS + lane;
        if (n >= N) continue;
        const uint8_t* blk = codes + (rb * NC + c) * TQ_B3_CHUNK_BYTES;
        const uint4 p0 = *reinterpret_cast<const uint4*>(blk + lane * 16);
        const uint4 p1 = *reinterpret_cast<const uint4*>(blk + 1024 + lane * 16);
        const uint2 p2 = *reinterpret_cast<const uint2*>(blk + 2048 + lane * 8);
        const uint32_t w[11] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w, p2.x, p2.y, 0u};
        for (int j = 0; j < 32; ++j) {
            const int bit = 10 * j, dw = bit >> 5, sh = bit & 31;
            uint32_t code = w[dw] >> sh;
            if (sh > 22) code |= w[dw + 1] << (32 - sh);
            code &= 0x3FFu;
            if (code >= (uint32_t)TQ_B3_CODES) code = 0;
            for (int h = 0; h < 2; ++h) {
                const int64_t col = c * TQ_CHUNK + 2 * j + h;
                if (col >= Kin) continue;
                const int u = (int)(h ? code / 27u : code % 27u);
                int v = u > 13 ? u - 27 : u;
                for (int k = 2; k >= 0; --k) {      // least significant digit first: plane 2
                    const int r = ((v % 3) + 3) % 3;
                    const int tv = r == 2 ? -1 : r;
                    trits[((int64_t)k * N + n) * Kin + col] = (int8_t)tv;
                    v = (v - tv) / 3;
                }
            }
        }
    }
}

// CODEBOOK: one thread per index dword (six groups of one row).
__global__ void k_pack_indices(const uint8_t* __restrict__ idx, uint32_t* __restrict__ out,
                               uint32_t* status, int64_t total, int64_t N, int64_t G, int64_t NID,
                               int ncb, int unpack, uint8_t* __restrict__ idx_out)
{
    uint32_t bad = 0;
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int lane = (int)(t & 63);
        const int64_t rest = t >> 6;
        const int64_t id = rest % NID;
        const int64_t rb = rest / NID;
        const int64_t n = rb * TQ_ROWS + lane;
        if (!unpack) {
            uint32_t w = 0;
            for (int j = 0; j < 6; ++j) {
                const int64_t grp = 6 * id + j;
                if (n < N && grp < G) {
                    const uint32_t v = idx[n * G + grp];
                    if ((int)v >= ncb) bad |= TQ_PACK_BAD_INDEX;
                    w |= (v & 31u) << (5 * j);
                }
            }
            out[t] = w;
        } else {
            const uint32_t w = out[t];
            for (int j = 0; j < 6; ++j) {
                const int64_t grp = 6 * id + j;
                if (n < N && grp < G) idx_out[n * G + grp] = (uint8_t)((w >> (5 * j)) & 31u);
            }
        }
    }
    if (bad) atomicOr(status, bad);
}

// Small copies with checks: TENSOR fp32 scales or the f16 codebook.
__global__ void k_pack_small(const void* __restrict__ src, void* __restrict__ dst, uint32_t* status,
                             int n, int slots, int is_f16, int unpack)
{
    const int i = threadIdx.x;
    if (i >= slots) return;
    if (is_f16) {
        const uint16_t* s = (const uint16_t*)src;
        uint16_t* d = (uint16_t*)dst;
        if (unpack) {
            if (i < n) d[i] = s[i];
        } else {
            const uint16_t v = i < n ? s[i] : 0;
            if (i < n && !f16_finite(v)) atomicOr(status, TQ_PACK_BAD_SCALE);
            d[i] = v;
        }
    } else {
        const float* s = (const float*)src;
        float* d = (float*)dst;
        if (unpack) {
            if (i < n) d[i] = s[i];
        } else {
            const float v = i < n ? s[i] : 0.0f;
            if (i < n && !isfinite(v)) atomicOr(status, TQ_PACK_BAD_SCALE);
            d[i] = v;
        }
    }
}

int grid_for(int64_t total)
{
    int64_t b = (total + kBlock - 1) / kBlock;
    const int64_t cap = (int64_t)tq_device_cus() * 64;
    if (b > cap) b = cap;
    return (int)(b < 1 ? 1 : b);
}

}  // namespace

TQ_EXPORT tq_status tq_pack(const tq_weight_desc* desc, const int8_t* trits, const void* scales,
                            const uint16_t* codebook, void* blob, void* stream_)
{
    tq_layout L;
    tq_status s = tq_check_desc(desc, &L);
    if (s) return s;
    const bool need_trits = L.N > 0 && L.Kin > 0;
    if ((s = tq_check_ptr(trits, "trits", !need_trits))) return s;
    if ((s = tq_check_ptr(scales, "scales", L.layout != TQ_SCALE_TENSOR && !need_trits, 4))) return s;
    if ((s = tq_check_ptr(blob, "blob", false))) return s;
    if (tq_is_codebook(L.layout)) {
        if ((s = tq_check_ptr(codebook, "codebook", false, 2))) return s;
    }
    hipStream_t stream = (hipStream_t)stream_;
    uint8_t* b = (uint8_t*)blob;
    uint32_t* status = (uint32_t*)(b + TQ_STATUS_OFFSET);
    // every byte of the blob is defined: padding and unused slots are zero
    if ((s = tq_check_hip(hipMemsetAsync(blob, 0, (size_t)L.total, stream), "tq_pack clear")))
        return s;
    hipLaunchKernelGGL(k_write_header, dim3(1), dim3(64), 0, stream, (tq_blob_header*)b, *desc);
    if ((s = tq_check_launch("tq_pack header"))) return s;
    const int64_t ncodes = L.codes_bytes / 4;
    if (ncodes > 0 && L.layout == TQ_SCALE_CODEBOOK_B3) {
        const int64_t n = L.NB * L.NC * TQ_ROWS;
        hipLaunchKernelGGL(k_pack_b3, dim3(grid_for(n)), dim3(kBlock), 0, stream, trits, b + L.codes_off, status, n,
                           L.N, L.Kin, L.NC);
        if ((s = tq_check_launch("tq_pack codes"))) return s;
    } else if (ncodes > 0) {
        hipLaunchKernelGGL(k_pack_codes, dim3(grid_for(ncodes)), dim3(kBlock), 0, stream, trits,
                           (uint32_t*)(b + L.codes_off), status, ncodes, L.K, L.N, L.Kin, L.NC);
        if ((s = tq_check_launch("tq_pack codes"))) return s;
    }
    if (L.layout == TQ_SCALE_TENSOR) {
        hipLaunchKernelGGL(k_pack_small, dim3(1), dim3(64), 0, stream, scales,
                           (void*)(b + L.scales_off), status, L.K, 64, 0, 0);
    } else if (L.layout == TQ_SCALE_GROUP_F16) {
        const int64_t n = L.scales_bytes / 4;
        if (n > 0)
            hipLaunchKernelGGL(k_pack_group_scales, dim3(grid_for(n)), dim3(kBlock), 0, stream,
                               (const uint16_t*)scales, (uint32_t*)(b + L.scales_off), status, n,
                               L.K, L.N, L.G, L.NGD, 0, (uint16_t*)nullptr);
    } else {
        hipLaunchKernelGGL(k_pack_small, dim3(1), dim3(64), 0, stream, (const void*)codebook,
                           (void*)(b + L.cb_off), status, L.ncb, TQ_CB_SLOTS, 1, 0);
        const int64_t n = L.scales_bytes / 4;
        if (n > 0)
            hipLaunchKernelGGL(k_pack_indices, dim3(grid_for(n)), dim3(kBlock), 0, stream,
                               (const uint8_t*)scales, (uint32_t*)(b + L.scales_off), status, n,
                               L.N, L.G, L.NID, L.ncb, 0, (uint8_t*)nullptr);
    }
    if ((s = tq_check_launch("tq_pack scales"))) return s;
    uint32_t host_status = 0;
    if ((s = tq_check_hip(hipMemcpyAsync(&host_status, status, 4, hipMemcpyDeviceToHost, stream),
                          "tq_pack status copy")))
        return s;
    if ((s = tq_check_hip(hipStreamSynchronize(stream), "tq_pack synchronize"))) return s;
    if (host_status)
        return tq_fail(TQ_ERR_VALUE, "tq_pack: invalid input (%s%s%s)",
                       host_status & TQ_PACK_BAD_TRIT ? "trit outside {-1,0,1} " : "",
                       host_status & TQ_PACK_BAD_SCALE ? "non-finite scale " : "",
                       host_status & TQ_PACK_BAD_INDEX ? "codebook index >= n_codebook" : "");
    return tq_ok();
}

TQ_EXPORT tq_status tq_unpack(const tq_weight_desc* desc, const void* blob, int8_t* trits,
                              void* scales, uint16_t* codebook, void* stream_)
{
    tq_layout L;
    tq_status s = tq_check_desc(desc, &L);
    if (s) return s;
    const bool need = L.N > 0 && L.Kin > 0;
    if ((s = tq_check_ptr(blob, "blob", false))) return s;
    if ((s = tq_check_ptr(trits, "trits", !need))) return s;
    if ((s = tq_check_ptr(scales, "scales", true, 4))) return s;
    if ((s = tq_check_ptr(codebook, "codebook", true, 2))) return s;
    hipStream_t stream = (hipStream_t)stream_;
    const uint8_t* b = (const uint8_t*)blob;
    const int64_t ncodes = L.codes_bytes / 4;
    if (ncodes > 0 && trits && L.layout == TQ_SCALE_CODEBOOK_B3) {
        const int64_t n = L.NB * L.NC * TQ_ROWS;
        hipLaunchKernelGGL(k_unpack_b3, dim3(grid_for(n)), dim3(kBlock), 0, stream, b + L.codes_off, trits, n, L.N,
                           L.Kin, L.NC);
        if ((s = tq_check_launch("tq_unpack codes"))) return s;
    } else if (ncodes > 0 && trits) {
        hipLaunchKernelGGL(k_unpack_codes, dim3(grid_for(ncodes)), dim3(kBlock), 0, stream,
                           (const uint32_t*)(b + L.codes_off), trits, ncodes, L.K, L.N, L.Kin, L.NC);
        if ((s = tq_check_launch("tq_unpack codes"))) return s;
    }
    if (scales) {
        if (L.layout == TQ_SCALE_TENSOR) {
            hipLaunchKernelGGL(k_pack_small, dim3(1), dim3(64), 0, stream,
                               (const void*)(b + L.scales_off), scales, (uint32_t*)nullptr, L.K,
                               L.K, 0, 1);
        } else if (L.layout == TQ_SCALE_GROUP_F16) {
            const int64_t n = L.scales_bytes / 4;
            if (n > 0)
                hipLaunchKernelGGL(k_pack_group_scales, dim3(grid_for(n)), dim3(kBlock), 0, stream,
                                   (const uint16_t*)nullptr, (uint32_t*)(b + L.scales_off),
                                   (uint32_t*)nullptr, n, L.K, L.N, L.G, L.NGD, 1, (uint16_t*)scales);
        } else {
            const int64_t n = L.scales_bytes / 4;
            if (n > 0)
                hipLaunchKernelGGL(k_pack_indices, dim3(grid_for(n)), dim3(kBlock), 0, stream,
                                   (const uint8_t*)nullptr, (uint32_t*)(b + L.scales_off),
                                   (uint32_t*)nullptr, n, L.N, L.G, L.NID, L.ncb, 1, (uint8_t*)scales);
        }
        if ((s = tq_check_launch("tq_unpack scales"))) return s;
    }
    if (codebook && tq_is_codebook(L.layout)) {
        hipLaunchKernelGGL(k_pack_small, dim3(1), dim3(64), 0, stream, (const void*)(b + L.cb_off),
                           (void*)codebook, (uint32_t*)nullptr, L.ncb, L.ncb, 1, 1);
        if ((s = tq_check_launch("tq_unpack codebook"))) return s;
    }
    return tq_ok();
}
