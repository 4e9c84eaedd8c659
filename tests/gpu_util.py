"""Helpers of the GPU tests: device transfers, packing through the C ABI, the
tolerance of the floating-point paths, and an independent reader of the
documented blob layout (written from the layout's description, sharing no
code with the library)."""
from __future__ import annotations

import numpy as np

TOL = 1e-3   # per token: max_n |y - y*| / max(|y*|, rms(y*))


def torch():
    import torch as t
    return t


def dev(a):
    """numpy -> cuda tensor (u16 travels as int16 bits)."""
    t = torch()
    a = np.ascontiguousarray(a)
    assert a.dtype != np.float64, "device arrays here are fp32 / bf16 / integer"
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return t.from_numpy(a).to("cuda")


def host(x, dtype=None):
    a = x.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def pack(K, g, layout, trits, scales, codebook=None, n_cb=27):
    from ternary_weight_amd import tq
    N, Kin = trits.shape[1], trits.shape[2]
    d = tq.desc(K, g, layout, N, Kin, n_codebook=(n_cb if layout == tq.SCALE_CODEBOOK else 0))
    blob = torch().empty(tq.packed_size(d), dtype=torch().uint8, device="cuda")
    tq.pack(d, dev(trits), dev(scales), None if codebook is None else dev(codebook), blob)
    return d, blob


def gemv(d, blob, x_type, x, x_scale=None, want_acc=False, gemm=False):
    from ternary_weight_amd import tq
    t = torch()
    M = x.shape[0]
    y = t.full((M, d.out_features), float("nan"), dtype=t.float32, device="cuda")
    acc = t.full((M, d.out_features), -12345, dtype=t.int32, device="cuda") if want_acc else None
    xd = x if isinstance(x, t.Tensor) else dev(x)
    xs = None if x_scale is None else (x_scale if isinstance(x_scale, t.Tensor) else dev(x_scale))
    (tq.gemm if gemm else tq.gemv)(d, blob, M, x_type, xd, xs, y, acc)
    t.cuda.synchronize()
    return (host(y), host(acc)) if want_acc else host(y)


def rel_err(y, ystar):
    """Per-token error metric of the floating-point paths (max over tokens)."""
    y = np.asarray(y, dtype=np.float64)
    ystar = np.asarray(ystar, dtype=np.float64)
    worst = 0.0
    for m in range(ystar.shape[0]):
        rms = np.sqrt(np.mean(ystar[m] ** 2)) if ystar.shape[1] else 0.0
        den = np.maximum(np.abs(ystar[m]), rms)
        den = np.where(den == 0, 1.0, den)
        if ystar.shape[1]:
            worst = max(worst, float(np.max(np.abs(y[m] - ystar[m]) / den)))
    return worst


# ---------------------------------------------------------------------------
# Reader of the documented blob layout.
# ---------------------------------------------------------------------------
def _align256(v):
    return (v + 255) & ~255


def b3_stream_codes(words):
    """The 32 ten-bit codes of 320-bit streams: words uint32 [..., 10] -> [..., 32]."""
    w = np.asarray(words, dtype=np.uint64)
    out = np.zeros(w.shape[:-1] + (32,), dtype=np.int64)
    for j in range(32):
        bit = 10 * j
        d, sh = bit // 32, bit % 32
        v = w[..., d] >> np.uint64(sh)
        if sh > 22:
            v = v | (w[..., d + 1] << np.uint64(32 - sh))
        out[..., j] = (v & np.uint64(0x3FF)).astype(np.int64)
    return out


def b3_digits(codes):
    """Pair codes -> the three digit planes of the two columns: int8 [3][..., 2]
    (codes >= 729 read as zero weights)."""
    codes = np.where(codes < 729, codes, 0)
    vals = np.stack([codes % 27, codes // 27], axis=-1)
    vals = np.where(vals > 13, vals - 27, vals)              # v in [-13, 13]
    digits = []
    for _ in range(3):                                        # least significant first
        r = np.mod(vals, 3)
        t = np.where(r == 2, -1, r)
        digits.append(t.astype(np.int8))
        vals = (vals - t) // 3
    return np.stack(digits[::-1], axis=0)                     # plane 0 = the most significant


def read_blob(blob, K, N, Kin, layout, g=0):
    """(trits int8 [K][N][Kin], raw 2-bit codes [K][NBr][NCc], scales, codebook)."""
    b = np.asarray(blob, dtype=np.uint8)
    NB, NC = (N + 63) // 64, (Kin + 63) // 64
    if layout == 3:
        return _read_b3(b, N, Kin, g, NB, NC)
    nwords = NB * NC * K * 64 * 4
    words = b[256:256 + 4 * nwords].view(np.uint32).reshape(NB, NC, K, 64, 4)
    d = np.arange(4).reshape(4, 1, 1)
    p = np.arange(4).reshape(1, 4, 1)
    bb = np.arange(4).reshape(1, 1, 4)
    shift = (8 * bb + 2 * p).astype(np.uint32)                       # [1,4,4] over (p, b)
    codes = (words[..., None, None] >> shift) & np.uint32(3)          # [NB,NC,K,64,4d,4p,4b]
    # column inside the chunk: 16d + 4p + b
    codes = codes.reshape(NB, NC, K, 64, 64)                           # (d,p,b) is row-major = col order
    codes = codes.transpose(2, 0, 3, 1, 4).reshape(K, NB * 64, NC * 64)
    trits = ((codes & 1).astype(np.int8) - (codes >> 1).astype(np.int8))
    out = {"codes": codes, "trits": trits[:, :N, :Kin]}
    end = _align256(256 + 4 * nwords)
    if layout == 0:
        out["scales"] = b[end:end + 4 * K].view(np.float32).copy()
    elif layout == 1:
        G = Kin // g
        NGD = (G + 1) // 2
        sw = b[end:end + NB * NGD * K * 64 * 4].view(np.uint32).reshape(NB, NGD, K, 64)
        halves = np.stack([sw & 0xFFFF, sw >> 16], axis=-1).astype(np.uint16)   # [NB,NGD,K,64,2]
        s = halves.transpose(2, 0, 3, 1, 4).reshape(K, NB * 64, NGD * 2)
        out["scales"] = s[:, :N, :G]
    else:
        G = Kin // g
        NID = (G + 5) // 6
        out["codebook"] = b[end:end + 64].view(np.uint16).copy()
        iw = b[end + 256:end + 256 + NB * NID * 64 * 4].view(np.uint32).reshape(NB, NID, 64)
        j = np.arange(6, dtype=np.uint32)
        idx = ((iw[..., None] >> (5 * j)) & np.uint32(31)).astype(np.uint8)      # [NB,NID,64,6]
        out["scales"] = idx.transpose(0, 2, 1, 3).reshape(NB * 64, NID * 6)[:N, :G]
    return out


def _read_b3(b, N, Kin, g, NB, NC):
    """The compact base-3 codec blob: per (row block, chunk) 2560 bytes -- the
    64 lanes' dwords 0..3, then 4..7 (16 bytes a lane), then 8..9 (8 bytes a
    lane) of each row's 320-bit stream; then the codebook and indices as for
    the codebook layout."""
    nbytes = NB * NC * 2560
    blk = b[256:256 + nbytes].reshape(NB, NC, 2560)
    p0 = blk[:, :, :1024].view(np.uint32).reshape(NB, NC, 64, 4)
    p1 = blk[:, :, 1024:2048].view(np.uint32).reshape(NB, NC, 64, 4)
    p2 = blk[:, :, 2048:].view(np.uint32).reshape(NB, NC, 64, 2)
    words = np.concatenate([p0, p1, p2], axis=-1)                     # [NB, NC, 64 lanes, 10]
    codes = b3_stream_codes(words)                                    # [NB, NC, 64, 32]
    digits = b3_digits(codes)                                         # [3, NB, NC, 64, 32, 2]
    trits = digits.reshape(3, NB, NC, 64, 64).transpose(0, 1, 3, 2, 4).reshape(3, NB * 64, NC * 64)
    codes_rc = codes.transpose(0, 2, 1, 3).reshape(NB * 64, NC * 32)
    out = {"codes": codes_rc, "trits": trits[:, :N, :Kin]}
    end = _align256(256 + nbytes)
    G = Kin // g
    NID = (G + 5) // 6
    out["codebook"] = b[end:end + 64].view(np.uint16).copy()
    iw = b[end + 256:end + 256 + NB * NID * 64 * 4].view(np.uint32).reshape(NB, NID, 64)
    j = np.arange(6, dtype=np.uint32)
    idx = ((iw[..., None] >> (5 * j)) & np.uint32(31)).astype(np.uint8)
    out["scales"] = idx.transpose(0, 2, 1, 3).reshape(NB * 64, NID * 6)[:N, :G]
    return out
