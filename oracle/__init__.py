"""CPU oracle of the packed ternary-weight product -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It loads ``liboracle.so`` (plain C,
built from ``oracle.c``) through ctypes and takes canonical numpy arrays; it
never sees the packed device layout and shares no code with the HIP library.

Every function here is argument marshalling only; the arithmetic and its
citations are in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

TENSOR, GROUP_F16, CODEBOOK = 0, 1, 2
F32, BF16, I8 = 0, 1, 2

_CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
           "-std=c99", "-Wall", "-Wextra"]


_SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def build(force: bool = False, sanitize: bool = False, out: str = "") -> str:
    """Compile liboracle.so with gcc (plain C, OpenMP over output rows).
    sanitize: AddressSanitizer and UndefinedBehaviorSanitizer, into `out`."""
    if sanitize:
        subprocess.check_call(["gcc", *_CFLAGS, *_SAN_FLAGS, SRC, "-o", out, "-lm"])
        return out
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_CFLAGS, SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


class OracleError(RuntimeError):
    pass


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _scales_dtype(layout):
    return {TENSOR: np.float32, GROUP_F16: np.uint16, CODEBOOK: np.uint8}[layout]


class Oracle:
    """ctypes view of one build of oracle.c (the default one, or a test's variant)."""

    def __init__(self, path: str):
        L = ctypes.CDLL(path)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.oracle_gemv_fp.argtypes = [i32, i32, i32, i32, i64, i64, vp, vp, vp, i64, i32, vp, vp, i32]
        L.oracle_gemv_fp.restype = i32
        L.oracle_gemv_i8.argtypes = [i32, i32, i32, i32, i64, i64, vp, vp, vp, i64, vp, vp,
                                     vp, vp, vp, i32]
        L.oracle_gemv_i8.restype = i32
        L.oracle_act_quant_i8.argtypes = [i64, i64, i32, vp, vp, vp]
        L.oracle_act_quant_i8.restype = i32
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f64.restype = ctypes.c_double
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_rms_norm.argtypes = [i64, vp, vp, ctypes.c_float, vp]
        L.oracle_rms_norm.restype = i32
        L.oracle_relu2_mul.argtypes = [i64, vp, vp, vp]
        L.oracle_relu2_mul.restype = i32
        L.oracle_bitnet_layer.argtypes = [i64, i64, i32, i32, i32, ctypes.c_float, vp, vp, vp, vp, vp, vp,
                                          vp, vp]
        L.oracle_bitnet_layer.restype = i32
        L.oracle_ternarize.argtypes = [i32, i32, i32, i32, i64, i64, vp, vp, vp, vp]
        L.oracle_ternarize.restype = i32
        L.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_f16.restype = ctypes.c_uint16
        L.oracle_threads.argtypes = []
        L.oracle_threads.restype = i32
        self.L = L
        self.path = path

    def gemv_fp(self, K, g, layout, trits, scales, x, x_type, codebook=None, nthreads=0):
        """fp64 y [M][N] for fp32 (x_type=F32) or bf16-bits (x_type=BF16) activations."""
        trits = _c(trits, np.int8)
        _, N, Kin = trits.shape
        scales = _c(scales, _scales_dtype(layout))
        codebook = _c(codebook, np.uint16)
        x = _c(x, np.float32 if x_type == F32 else np.uint16).reshape(-1, Kin)
        M = x.shape[0]
        y = np.zeros((M, N), dtype=np.float64)
        ncb = 0 if codebook is None else len(codebook)
        rc = self.L.oracle_gemv_fp(K, g, layout, ncb, N, Kin, _p(trits), _p(scales),
                                   _p(codebook), M, x_type, _p(x), _p(y), nthreads)
        if rc:
            raise OracleError("oracle_gemv_fp failed with status %d" % rc)
        return y

    def act_quant_i8(self, x, x_type=F32):
        """(q int8 [M][Kin], s fp32 [M]) by the per-token absmax rule."""
        x = _c(x, np.float32 if x_type == F32 else np.uint16)
        x = x.reshape(-1, x.shape[-1])
        M, Kin = x.shape
        q = np.zeros((M, Kin), dtype=np.int8)
        s = np.zeros(M, dtype=np.float32)
        rc = self.L.oracle_act_quant_i8(M, Kin, x_type, _p(x), _p(q), _p(s))
        if rc:
            raise OracleError("oracle_act_quant_i8 failed with status %d" % rc)
        return q, s

    def gemv_i8(self, K, g, layout, trits, scales, xq, xs, codebook=None, want_y32=None,
                nthreads=0):
        """dict(acc int64 [M][N], y64 fp64 [M][N], y32 fp32 [M][N] or None)."""
        trits = _c(trits, np.int8)
        _, N, Kin = trits.shape
        scales = _c(scales, _scales_dtype(layout))
        codebook = _c(codebook, np.uint16)
        xq = _c(xq, np.int8).reshape(-1, Kin)
        xs = _c(xs, np.float32).reshape(-1)
        M = xq.shape[0]
        acc = np.zeros((M, N), dtype=np.int64)
        y64 = np.zeros((M, N), dtype=np.float64)
        if want_y32 is None:
            want_y32 = layout == TENSOR and K == 1
        y32 = np.zeros((M, N), dtype=np.float32) if want_y32 else None
        ncb = 0 if codebook is None else len(codebook)
        rc = self.L.oracle_gemv_i8(K, g, layout, ncb, N, Kin, _p(trits), _p(scales),
                                   _p(codebook), M, _p(xq), _p(xs), _p(acc), _p(y64), _p(y32),
                                   nthreads)
        if rc:
            raise OracleError("oracle_gemv_i8 failed with status %d" % rc)
        return {"acc": acc, "y64": y64, "y32": y32}

    def rms_norm(self, x, w, eps):
        """fp32 RMSNorm of the vector x with weight w."""
        x, w = _c(x, np.float32).reshape(-1), _c(w, np.float32).reshape(-1)
        out = np.zeros_like(x)
        rc = self.L.oracle_rms_norm(len(x), _p(x), _p(w), float(eps), _p(out))
        if rc:
            raise OracleError("oracle_rms_norm failed with status %d" % rc)
        return out

    def relu2_mul(self, g, u):
        g, u = _c(g, np.float32).reshape(-1), _c(u, np.float32).reshape(-1)
        out = np.zeros_like(g)
        rc = self.L.oracle_relu2_mul(len(g), _p(g), _p(u), _p(out))
        if rc:
            raise OracleError("oracle_relu2_mul failed with status %d" % rc)
        return out

    def bitnet_layer(self, dims, trits, s_w, norms, x):
        """One decode-chain layer for the first token.

        dims: (hidden, inter, n_heads, n_kv, head_dim, eps); trits: 7 int8
        [N][Kin] arrays (q, k, v, o, gate, up, down); s_w: their 7 fp32
        scales; norms: (input, attention-sub, post-attention, FFN-sub) fp32
        weights.  Returns (x after the layer, q|k|v fp32)."""
        hidden, inter, nh, nkv, hd, eps = dims
        ts = [_c(t, np.int8).reshape(t.shape[-2], t.shape[-1]) for t in trits]
        ptrs = (ctypes.c_void_p * 7)(*[t.ctypes.data for t in ts])
        sw = np.ascontiguousarray(s_w, dtype=np.float32)
        ns = [_c(n, np.float32) for n in norms]
        x = np.array(x, dtype=np.float32).reshape(-1)
        qkv = np.zeros((nh + 2 * nkv) * hd, dtype=np.float32)
        rc = self.L.oracle_bitnet_layer(hidden, inter, nh, nkv, hd, float(eps), ctypes.cast(ptrs, ctypes.c_void_p),
                                        _p(sw), _p(ns[0]), _p(ns[1]), _p(ns[2]), _p(ns[3]), _p(x), _p(qkv))
        if rc:
            raise OracleError("oracle_bitnet_layer failed with status %d" % rc)
        return x, qkv

    def ternarize(self, K, g, layout, w, codebook=None):
        """(trits int8 [K][N][Kin], canonical scales) fitted to the fp32 weight w [N][Kin]."""
        w = _c(w, np.float32)
        N, Kin = w.shape
        codebook = _c(codebook, np.uint16)
        ncb = 0 if codebook is None else len(codebook)
        trits = np.zeros((K, N, Kin), dtype=np.int8)
        if layout == TENSOR:
            scales = np.zeros(K, dtype=np.float32)
        elif layout == GROUP_F16:
            scales = np.zeros((K, N, Kin // g), dtype=np.uint16)
        else:
            scales = np.zeros((N, Kin // g), dtype=np.uint8)
        rc = self.L.oracle_ternarize(K, g, layout, ncb, N, Kin, _p(w), _p(codebook), _p(trits), _p(scales))
        if rc:
            raise OracleError("oracle_ternarize failed with status %d" % rc)
        return trits, scales

    def f32_to_f16(self, f: float) -> int:
        return self.L.oracle_f32_to_f16(float(f))

    def f16_to_f64(self, h: int) -> float:
        return self.L.oracle_f16_to_f64(int(h))

    def bf16_to_f32(self, b: int) -> float:
        return self.L.oracle_bf16_to_f32(int(b))

    def threads(self) -> int:
        return self.L.oracle_threads()


_default = None


def default() -> Oracle:
    """The oracle build the tests use (TQ_ORACLE_LIB names another build, e.g.
    a sanitizer one)."""
    global _default
    if _default is None:
        _default = Oracle(os.environ.get("TQ_ORACLE_LIB") or build())
    return _default


def gemv_fp(*a, **k):
    return default().gemv_fp(*a, **k)


def gemv_i8(*a, **k):
    return default().gemv_i8(*a, **k)


def act_quant_i8(*a, **k):
    return default().act_quant_i8(*a, **k)


def rms_norm(*a, **k):
    return default().rms_norm(*a, **k)


def relu2_mul(*a, **k):
    return default().relu2_mul(*a, **k)


def bitnet_layer(*a, **k):
    return default().bitnet_layer(*a, **k)


def ternarize(*a, **k):
    return default().ternarize(*a, **k)


def f16_to_f64(h: int) -> float:
    return default().f16_to_f64(h)


def bf16_to_f32(b: int) -> float:
    return default().bf16_to_f32(b)


def threads() -> int:
    return default().threads()
