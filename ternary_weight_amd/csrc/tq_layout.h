// Packed blob layout of libtq (host and device).
//
// A blob is one weight N x Kin with K trit planes and its scales:
//
//   [0, 256)        header: magic "TQW1", format version, desc fields, and the
//                   pack status word at byte 64 (set by tq_pack's checks)
//   codes           trit planes, 2 bits per trit, four trits per byte
//   scale region    TENSOR: K fp32 | GROUP_F16: f16 pairs | CODEBOOK: 32-entry
//                   f16 codebook then 5-bit group indices
//
// Codes.  Rows are taken in blocks of 64 (one row per lane of a wave64) and
// columns in chunks of 64.  For row block rb, column chunk c and plane k the
// 64 lanes' 16-byte slots are contiguous (1 KiB, one coalesced 128-bit load
// per lane):
//     slot(k, rb, c, lane) = codes + (((rb * NC + c) * K + k) * 64 + lane) * 16
// The slot holds columns c*64 .. c*64+63 of row rb*64 + lane in four dwords;
// dword d holds the 16 columns 16d .. 16d+15 and column 16d + 4p + b sits in
// byte b, bits 2p and 2p+1.  So (dword >> 2p) & 0x03030303 gives the codes of
// four consecutive columns 16d+4p .. 16d+4p+3, one per byte.  Codes: 00 = 0,
// 01 = +1, 10 = -1; 11 is never written and decodes to 0.
// Rows beyond N and columns beyond Kin are padding with code 00.
//
// GROUP_F16 scales: one dword per (row block, pair of groups, plane, lane),
//     dword(rb, gd, k, lane) = scales + (((rb * NGD + gd) * K + k) * 64 + lane) * 4
// with group 2gd in the low half and 2gd+1 in the high half (f16 bits).
//
// CODEBOOK: 32 f16 codebook entries (64 bytes, unused entries 0) at cb_off,
// then one dword per (row block, six groups, lane),
//     dword(rb, id, lane) = idx + ((rb * NID + id) * 64 + lane) * 4
// holding the 5-bit index of group 6id + j in bits 5j .. 5j+4 (j = 0..5).
//
// TENSOR: K fp32 scales at scales_off.
//
// CODEBOOK_B3 (the codec with compact base-3 codes; K = 3 digits): the
// codebook and the 5-bit group indices as CODEBOOK, and in place of the K
// two-bit planes one 320-bit stream per (row, 64-column chunk): the weights'
// base-27 values v = 9 t0 + 3 t1 + t2 (digit planes 0, 1, 2), two columns per
// 10-bit code
//     code(j) = (v[2j] mod 27) + 27 (v[2j+1] mod 27)       j = 0 .. 31
// at bits 10j .. 10j+9 of the stream (little-endian dwords 0..9, so the
// 16-column unit d is bits 80d .. 80d+79).  Code 0 is two zero weights;
// codes 729 .. 1023 are never written and read as zeros.  For row block rb
// and chunk c the 64 lanes' streams are stored in three parts, 2560 bytes:
//     dwords 0..3: codes + (rb * NC + c) * 2560 +        lane * 16
//     dwords 4..7: codes + (rb * NC + c) * 2560 + 1024 + lane * 16
//     dwords 8..9: codes + (rb * NC + c) * 2560 + 2048 + lane * 8
// so a wave reads its chunk with two 1 KiB and one 512-byte coalesced load.
#pragma once

#include <stdint.h>

#include "../../include/tq.h"

#define TQ_BLOB_MAGIC 0x31575154u   // "TQW1" little-endian
#define TQ_BLOB_VERSION 1u
#define TQ_HEADER_BYTES 256
#define TQ_STATUS_OFFSET 64         // uint32 pack status inside the header
#define TQ_ROWS 64                  // rows per block (lanes of a wave)
#define TQ_CHUNK 64                 // columns per 16-byte lane slot
#define TQ_MAX_KIN 65536
#define TQ_MAX_N (1 << 24)
#define TQ_MAX_M_GEMV 16
// Tokens the multi-token decode kernels take in one pass over the codes
// (more are taken in slices of this many).
#define TQ_PASS_TOKENS 4
#define TQ_CB_SLOTS 32
#define TQ_B3_CHUNK_BYTES 2560      // CODEBOOK_B3: bytes of one (row block, 64-column chunk)
#define TQ_B3_CODES 729             // CODEBOOK_B3: valid 10-bit pair codes (27 * 27)

// CODEBOOK and CODEBOOK_B3 share the codebook and the group indices.
#if defined(__HIP__)
__host__ __device__
#endif
static inline bool tq_is_codebook(int layout) { return layout == TQ_SCALE_CODEBOOK || layout == TQ_SCALE_CODEBOOK_B3; }

// pack status bits
#define TQ_PACK_BAD_TRIT 1u
#define TQ_PACK_BAD_SCALE 2u
#define TQ_PACK_BAD_INDEX 4u

struct tq_blob_header {
    uint32_t magic;
    uint32_t version;
    int32_t planes;
    int32_t group;
    int32_t scale_layout;
    int32_t n_codebook;
    int64_t out_features;
    int64_t in_features;
    uint32_t reserved0[6];
    uint32_t pack_status;           // byte 64
    uint32_t reserved1[47];
};
static_assert(sizeof(tq_blob_header) == TQ_HEADER_BYTES, "header size");
static_assert(__builtin_offsetof(tq_blob_header, pack_status) == TQ_STATUS_OFFSET, "status offset");

struct tq_layout {
    int64_t N, Kin;
    int32_t K, g, layout, ncb;
    int64_t NB;          // row blocks
    int64_t NC;          // column chunks
    int64_t G;           // groups per row (1 for TENSOR)
    int64_t NGD;         // GROUP_F16: group pairs per row
    int64_t NID;         // CODEBOOK: index dwords per row
    int64_t codes_off, codes_bytes;
    int64_t scales_off, scales_bytes;   // TENSOR / GROUP_F16 scales, CODEBOOK indices
    int64_t cb_off;                      // CODEBOOK codebook
    int64_t total;
};

static inline int64_t tq_align256(int64_t v) { return (v + 255) & ~(int64_t)255; }

static inline void tq_layout_make(const tq_weight_desc* d, tq_layout* L)
{
    L->N = d->out_features;
    L->Kin = d->in_features;
    L->K = d->planes;
    L->layout = d->scale_layout;
    L->g = (d->scale_layout == TQ_SCALE_TENSOR) ? 0 : d->group;
    L->ncb = tq_is_codebook(d->scale_layout) ? d->n_codebook : 0;
    L->NB = (L->N + TQ_ROWS - 1) / TQ_ROWS;
    L->NC = (L->Kin + TQ_CHUNK - 1) / TQ_CHUNK;
    L->G = (L->layout == TQ_SCALE_TENSOR) ? 1 : (L->g > 0 ? L->Kin / L->g : 0);
    L->NGD = (L->G + 1) / 2;
    L->NID = (L->G + 5) / 6;
    L->codes_off = TQ_HEADER_BYTES;
    L->codes_bytes = L->layout == TQ_SCALE_CODEBOOK_B3 ? L->NB * L->NC * TQ_B3_CHUNK_BYTES
                                                       : L->NB * L->NC * (int64_t)L->K * TQ_ROWS * 16;
    int64_t end = tq_align256(L->codes_off + L->codes_bytes);
    L->cb_off = 0;
    if (L->layout == TQ_SCALE_TENSOR) {
        L->scales_off = end;
        L->scales_bytes = 256;
    } else if (L->layout == TQ_SCALE_GROUP_F16) {
        L->scales_off = end;
        L->scales_bytes = L->NB * L->NGD * (int64_t)L->K * TQ_ROWS * 4;
    } else {
        L->cb_off = end;
        L->scales_off = end + 256;
        L->scales_bytes = L->NB * L->NID * TQ_ROWS * 4;
    }
    L->total = tq_align256(L->scales_off + L->scales_bytes);
}
