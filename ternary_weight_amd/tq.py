"""Python binding of libtq.so (include/tq.h): argument marshalling only.

Each function takes torch tensors that live on the GPU (or plain integers)
and passes their device pointers and the current HIP stream to the C call of
the same name; every step of the computation runs in the library's HIP
kernels.  A non-OK status raises ``TQError`` carrying ``tq_last_error()``.
The library must have been built (``python -m ternary_weight_amd.build``);
loading fails loudly otherwise -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# TQ_LIB names another build of the library (e.g. the sanitizer build of its host code)
LIB_PATH = os.environ.get("TQ_LIB") or os.path.join(PKG, "libtq.so")

OK, ERR_ARG, ERR_SHAPE, ERR_ALIGN, ERR_VALUE, ERR_UNSUPPORTED, ERR_DEVICE = range(7)
SCALE_TENSOR, SCALE_GROUP_F16, SCALE_CODEBOOK, SCALE_CODEBOOK_B3 = 0, 1, 2, 3
F32, BF16, I8, F32_Q8 = 0, 1, 2, 3


class TQError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        super().__init__("%s: %s (%d): %s" % (func, STATUS_NAMES.get(status, "?"), status, detail))
        self.status = status


STATUS_NAMES = {OK: "TQ_OK", ERR_ARG: "TQ_ERR_ARG", ERR_SHAPE: "TQ_ERR_SHAPE",
                ERR_ALIGN: "TQ_ERR_ALIGN", ERR_VALUE: "TQ_ERR_VALUE",
                ERR_UNSUPPORTED: "TQ_ERR_UNSUPPORTED", ERR_DEVICE: "TQ_ERR_DEVICE"}


class tq_weight_desc(ctypes.Structure):
    _fields_ = [("planes", ctypes.c_int32), ("group", ctypes.c_int32),
                ("scale_layout", ctypes.c_int32), ("n_codebook", ctypes.c_int32),
                ("out_features", ctypes.c_int64), ("in_features", ctypes.c_int64)]


class tq_problem(ctypes.Structure):
    _fields_ = [("desc", ctypes.POINTER(tq_weight_desc)), ("blob", ctypes.c_void_p),
                ("x", ctypes.c_void_p), ("x_scale", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("acc", ctypes.c_void_p)]


class tq_act_segment(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("in_features", ctypes.c_int64), ("x_type", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("x", ctypes.c_void_p), ("xq", ctypes.c_void_p),
                ("x_scale", ctypes.c_void_p)]


class tq_grouped_plan(ctypes.Structure):
    _fields_ = [("workspace", ctypes.c_void_p), ("n_items", ctypes.c_int64),
                ("family", ctypes.c_int32), ("x_type", ctypes.c_int32), ("M", ctypes.c_int32),
                ("waves", ctypes.c_int32), ("row_blocks", ctypes.c_int32),
                ("n_problems", ctypes.c_int32), ("x_lds_bytes", ctypes.c_int32),
                ("mode", ctypes.c_int32)]


class tq_bitnet_dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("intermediate", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("eps", ctypes.c_float)]


class tq_bitnet_layer(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p * 7), ("norm", ctypes.c_void_p * 4)]


class tq_chain_plan(ctypes.Structure):
    _fields_ = [("workspace", ctypes.c_void_p), ("n_layers", ctypes.c_int32),
                ("workgroups", ctypes.c_int32), ("dims", tq_bitnet_dims), ("reserved", ctypes.c_int32 * 4)]


# Every symbol the header declares, with its ctypes signature.
_VP, _I32, _I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
_DESC = ctypes.POINTER(tq_weight_desc)
SIGNATURES = {
    "tq_abi_version": ([], _I32),
    "tq_status_string": ([_I32], ctypes.c_char_p),
    "tq_last_error": ([], ctypes.c_char_p),
    "tq_packed_size": ([_DESC, ctypes.POINTER(ctypes.c_size_t)], _I32),
    "tq_pack": ([_DESC, _VP, _VP, _VP, _VP, _VP], _I32),
    "tq_unpack": ([_DESC, _VP, _VP, _VP, _VP, _VP], _I32),
    "tq_act_quant_int8": ([_I64, _I64, _I32, _VP, _VP, _VP, _VP], _I32),
    "tq_act_quant_int8_batch": ([ctypes.POINTER(tq_act_segment), _I32, _VP], _I32),
    "tq_gemv": ([_DESC, _VP, _I64, _I32, _VP, _VP, _VP, _VP, _VP], _I32),
    "tq_gemm": ([_DESC, _VP, _I64, _I32, _VP, _VP, _VP, _VP, _VP], _I32),
    "tq_gemv_grouped_workspace_size": ([ctypes.POINTER(tq_problem), _I32, _I64,
                                        ctypes.POINTER(ctypes.c_size_t)], _I32),
    "tq_gemv_grouped_prepare": ([ctypes.POINTER(tq_problem), _I32, _I64, _I32, _VP,
                                 ctypes.c_size_t, ctypes.POINTER(tq_grouped_plan), _VP], _I32),
    "tq_gemv_grouped_prepare_tokens": ([ctypes.POINTER(tq_problem), ctypes.POINTER(_I32), _I32, _I32, _VP,
                                        ctypes.c_size_t, ctypes.POINTER(tq_grouped_plan), _VP], _I32),
    "tq_gemv_grouped_run": ([ctypes.POINTER(tq_grouped_plan), _VP], _I32),
    "tq_gemm_grouped_workspace_size": ([ctypes.POINTER(tq_problem), _I32, _I64, _I32,
                                        ctypes.POINTER(ctypes.c_size_t)], _I32),
    "tq_gemm_grouped_prepare": ([ctypes.POINTER(tq_problem), _I32, _I64, _I32, _VP,
                                 ctypes.c_size_t, ctypes.POINTER(tq_grouped_plan), _VP], _I32),
    "tq_gemm_grouped_run": ([ctypes.POINTER(tq_grouped_plan), _VP], _I32),
    "tq_ternarize_workspace_size": ([_DESC, ctypes.POINTER(ctypes.c_size_t)], _I32),
    "tq_ternarize": ([_DESC, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP], _I32),
    "tq_ternarize_noalloc": ([_DESC, _VP, _VP, _VP, _VP, _VP], _I32),
    "tq_bitnet_chain_workspace_size": ([ctypes.POINTER(tq_bitnet_dims), _I32, ctypes.POINTER(ctypes.c_size_t)],
                                       _I32),
    "tq_bitnet_chain_prepare": ([ctypes.POINTER(tq_bitnet_dims), ctypes.POINTER(tq_bitnet_layer), _I32, _VP,
                                 ctypes.c_size_t, ctypes.POINTER(tq_chain_plan), _VP], _I32),
    "tq_bitnet_chain_run": ([ctypes.POINTER(tq_chain_plan), _VP, _VP, _VP], _I32),
    "tq_bitnet_chain_status": ([ctypes.POINTER(tq_chain_plan), _VP], _I32),
}

_lib = None


def lib():
    """Load libtq.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libtq.so is not built (%s); run `python -m ternary_weight_amd.build`"
                               % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(status: int, func: str):
    if status != OK:
        raise TQError(status, func, lib().tq_last_error().decode())


def _ptr(t):
    """Device pointer of a tensor (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def desc(planes: int, group: int, scale_layout: int, out_features: int, in_features: int,
         n_codebook: int = 0) -> tq_weight_desc:
    return tq_weight_desc(planes, group, scale_layout, n_codebook, out_features, in_features)


def abi_version() -> int:
    return lib().tq_abi_version()


def status_string(s: int) -> str:
    return lib().tq_status_string(s).decode()


def last_error() -> str:
    return lib().tq_last_error().decode()


def packed_size(d: tq_weight_desc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().tq_packed_size(ctypes.byref(d), ctypes.byref(n)), "tq_packed_size")
    return n.value


def pack(d, trits, scales, codebook, blob, stream=None):
    _check(lib().tq_pack(ctypes.byref(d), _ptr(trits), _ptr(scales), _ptr(codebook), _ptr(blob),
                         _stream(stream)), "tq_pack")


def unpack(d, blob, trits, scales, codebook=None, stream=None):
    _check(lib().tq_unpack(ctypes.byref(d), _ptr(blob), _ptr(trits), _ptr(scales),
                           _ptr(codebook), _stream(stream)), "tq_unpack")


def act_quant_int8(M, in_features, x_type, x, xq, x_scale, stream=None):
    _check(lib().tq_act_quant_int8(M, in_features, x_type, _ptr(x), _ptr(xq), _ptr(x_scale),
                                   _stream(stream)), "tq_act_quant_int8")


def act_quant_int8_batch(segments, stream=None):
    """segments: (M, in_features, x_type, x, xq, x_scale) tuples, one launch for all."""
    arr = (tq_act_segment * max(len(segments), 1))()
    for i, (M, kin, xt, x, xq, xs) in enumerate(segments):
        arr[i] = tq_act_segment(M, kin, xt, 0, _ptr(x), _ptr(xq), _ptr(xs))
    _check(lib().tq_act_quant_int8_batch(arr, len(segments), _stream(stream)), "tq_act_quant_int8_batch")


def gemv(d, blob, M, x_type, x, x_scale, y, acc=None, stream=None):
    _check(lib().tq_gemv(ctypes.byref(d), _ptr(blob), M, x_type, _ptr(x), _ptr(x_scale), _ptr(y),
                         _ptr(acc), _stream(stream)), "tq_gemv")


def gemm(d, blob, M, x_type, x, x_scale, y, acc=None, stream=None):
    _check(lib().tq_gemm(ctypes.byref(d), _ptr(blob), M, x_type, _ptr(x), _ptr(x_scale), _ptr(y),
                         _ptr(acc), _stream(stream)), "tq_gemm")


def problems(items):
    """ctypes array of tq_problem from (desc, blob, x, x_scale, y, acc) tuples.

    The descs must stay alive as long as the returned array is used."""
    arr = (tq_problem * len(items))()
    for i, (d, blob, x, xs, y, acc) in enumerate(items):
        arr[i] = tq_problem(ctypes.pointer(d), _ptr(blob), _ptr(x), _ptr(xs), _ptr(y), _ptr(acc))
    return arr


def gemv_grouped_workspace_size(probs, M) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().tq_gemv_grouped_workspace_size(probs, len(probs), M, ctypes.byref(n)),
           "tq_gemv_grouped_workspace_size")
    return n.value


def gemv_grouped_prepare(probs, M, x_type, workspace, workspace_bytes, waves=0, row_blocks=0,
                         stream=None):
    plan = tq_grouped_plan()
    plan.waves = waves
    plan.row_blocks = row_blocks
    _check(lib().tq_gemv_grouped_prepare(probs, len(probs), M, x_type, _ptr(workspace),
                                         workspace_bytes, ctypes.byref(plan), _stream(stream)),
           "tq_gemv_grouped_prepare")
    return plan


def gemv_grouped_prepare_tokens(probs, tokens, x_type, workspace, workspace_bytes, waves=0, row_blocks=0,
                                stream=None):
    """Grouped decode plan where problem i has its own token count tokens[i] (0..16)."""
    if len(tokens) != len(probs):
        raise ValueError("one token count per problem")
    counts = (_I32 * max(len(tokens), 1))(*[int(t) for t in tokens])
    plan = tq_grouped_plan()
    plan.waves = waves
    plan.row_blocks = row_blocks
    _check(lib().tq_gemv_grouped_prepare_tokens(probs, counts, len(probs), x_type, _ptr(workspace),
                                                workspace_bytes, ctypes.byref(plan), _stream(stream)),
           "tq_gemv_grouped_prepare_tokens")
    return plan


def gemv_grouped_run(plan, stream=None):
    _check(lib().tq_gemv_grouped_run(ctypes.byref(plan), _stream(stream)), "tq_gemv_grouped_run")


def gemm_grouped_workspace_size(probs, M, x_type) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().tq_gemm_grouped_workspace_size(probs, len(probs), M, x_type, ctypes.byref(n)),
           "tq_gemm_grouped_workspace_size")
    return n.value


def gemm_grouped_prepare(probs, M, x_type, workspace, workspace_bytes, stream=None):
    plan = tq_grouped_plan()
    _check(lib().tq_gemm_grouped_prepare(probs, len(probs), M, x_type, _ptr(workspace),
                                         workspace_bytes, ctypes.byref(plan), _stream(stream)),
           "tq_gemm_grouped_prepare")
    return plan


def gemm_grouped_run(plan, stream=None):
    _check(lib().tq_gemm_grouped_run(ctypes.byref(plan), _stream(stream)), "tq_gemm_grouped_run")


def bitnet_dims(hidden: int, intermediate: int, n_heads: int, n_kv_heads: int, head_dim: int,
                eps: float) -> tq_bitnet_dims:
    return tq_bitnet_dims(hidden, intermediate, n_heads, n_kv_heads, head_dim, eps)


def bitnet_chain_workspace_size(dims: tq_bitnet_dims, n_layers: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().tq_bitnet_chain_workspace_size(ctypes.byref(dims), n_layers, ctypes.byref(n)),
           "tq_bitnet_chain_workspace_size")
    return n.value


def bitnet_chain_prepare(dims: tq_bitnet_dims, layers, workspace, workspace_bytes, workgroups=0, stream=None):
    """layers: one (7 blobs q, k, v, o, gate, up, down; 4 norm weights) pair per layer."""
    arr = (tq_bitnet_layer * len(layers))()
    for i, (ws, ns) in enumerate(layers):
        for p in range(7):
            arr[i].w[p] = _ptr(ws[p])
        for j in range(4):
            arr[i].norm[j] = _ptr(ns[j])
    plan = tq_chain_plan()
    plan.workgroups = workgroups
    _check(lib().tq_bitnet_chain_prepare(ctypes.byref(dims), arr, len(layers), _ptr(workspace), workspace_bytes,
                                         ctypes.byref(plan), _stream(stream)), "tq_bitnet_chain_prepare")
    return plan


def bitnet_chain_run(plan, x, qkv=None, stream=None):
    _check(lib().tq_bitnet_chain_run(ctypes.byref(plan), _ptr(x), _ptr(qkv), _stream(stream)), "tq_bitnet_chain_run")


def bitnet_chain_status(plan, stream=None):
    _check(lib().tq_bitnet_chain_status(ctypes.byref(plan), _stream(stream)), "tq_bitnet_chain_status")


def ternarize_workspace_size(d: tq_weight_desc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().tq_ternarize_workspace_size(ctypes.byref(d), ctypes.byref(n)), "tq_ternarize_workspace_size")
    return n.value


def ternarize(d: tq_weight_desc, w, trits, scales, codebook=None, workspace=None, workspace_bytes=0, stream=None):
    _check(lib().tq_ternarize(ctypes.byref(d), _ptr(w), _ptr(codebook), _ptr(trits), _ptr(scales), _ptr(workspace),
                              workspace_bytes, _stream(stream)), "tq_ternarize")


def ternarize_noalloc(d: tq_weight_desc, w, trits, scales, codebook=None, stream=None):
    """tq_ternarize without a workspace: the library's own scratch array (no allocation)."""
    _check(lib().tq_ternarize_noalloc(ctypes.byref(d), _ptr(w), _ptr(codebook), _ptr(trits), _ptr(scales),
                                      _stream(stream)), "tq_ternarize_noalloc")
