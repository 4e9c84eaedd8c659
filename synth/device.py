"""GPU side of the input generator: fills torch tensors in HBM with exactly the
values synth.gen / synth.inputs produce on the host (test and benchmark
infrastructure; loads synth/libtqsynth.so)."""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import gen
from .configs import BF16, CODEBOOK, F32, GROUP_F16, I8

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtqsynth.so")

K_TRITS, K_DIGITS, K_INDICES, K_NORMAL_F32, K_NORMAL_BF16, K_LOGU_F16, K_LOGU_F32, K_NORMAL_F64 = range(8)

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libtqsynth.so is not built; run `python -m ternary_weight_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.synth_fill.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64,
                                 ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_void_p,
                                 ctypes.c_void_p]
        L.synth_fill.restype = ctypes.c_int
        L.synth_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_void_p]
        L.synth_stream_read.restype = ctypes.c_int
        _lib = L
    return _lib


def fill(kind: int, seed: int, start: int, out, a: float = 0.0, b: float = 0.0, div: float = 1.0,
         stream=None):
    import torch
    st = torch.cuda.current_stream().cuda_stream if stream is None else stream
    rc = lib().synth_fill(kind, seed & gen.MASK64, start, out.numel(), a, b, div, out.data_ptr(), st)
    if rc:
        raise RuntimeError("synth_fill failed: hip error %d" % rc)
    return out


def stream_read(buf, out, blocks: int = 0, stream=None):
    """Launch the plain streaming-read kernel over a whole uint8 buffer."""
    import torch
    st = torch.cuda.current_stream().cuda_stream if stream is None else stream
    rc = lib().synth_stream_read(buf.data_ptr(), buf.numel() // 16 * 16, out.data_ptr(), blocks, st)
    if rc:
        raise RuntimeError("synth_stream_read failed: hip error %d" % rc)


def projection(case, layer: int, proj: int, N: int, Kin: int, M=None, device="cuda"):
    """Device tensors with the same values as synth.inputs.projection(...)."""
    import torch
    from . import inputs
    s = inputs.seeds(case.cfg, layer, proj)
    K, g = case.planes, case.group
    M = case.M if M is None else M
    d = {"K": K, "g": g, "layout": case.layout, "N": N, "Kin": Kin, "M": M, "x_type": case.x_type}
    trits = torch.empty((K, N, Kin), dtype=torch.int8, device=device)
    if case.layout == CODEBOOK:
        fill(K_DIGITS, s["digits"], 0, trits)
        idx = torch.empty((N, Kin // g), dtype=torch.uint8, device=device)
        fill(K_INDICES, s["index"], 0, idx, a=float(inputs.N_CODEBOOK))
        d["scales"] = idx
        d["codebook"] = torch.from_numpy(gen.codebook_f16(inputs.N_CODEBOOK).view(np.int16)).to(device)
    else:
        fill(K_TRITS, s["trits"], 0, trits)
        lo, span = gen.log_uniform_params(1e-3, 1e-1)
        if case.layout == GROUP_F16:
            G = Kin // g
            sc = torch.empty((K, N, G), dtype=torch.int16, device=device)
            for k in range(K):
                fill(K_LOGU_F16, s["scales"], k * N * G, sc[k], a=lo, b=span, div=float(3 ** k))
            d["scales"] = sc
        else:
            sc = torch.empty((K,), dtype=torch.float32, device=device)
            fill(K_LOGU_F32, s["scales"], 0, sc, a=lo, b=span)
            d["scales"] = sc
        d["codebook"] = None
    d["trits"] = trits
    if case.x_type == BF16:
        x = torch.empty((M, Kin), dtype=torch.int16, device=device)
        fill(K_NORMAL_BF16, s["x"], 0, x)
    else:
        x = torch.empty((M, Kin), dtype=torch.float32, device=device)
        fill(K_NORMAL_F32, s["x"], 0, x)
    d["x"] = x
    return d


def moe_projection(moe, layer: int, expert: int, proj: int, device="cuda"):
    """Device tensors with the same values as synth.inputs.moe_projection(...)."""
    _, N, Kin = moe.proj_shapes()[proj]
    return projection(moe.case(), layer, expert * 3 + proj, N, Kin, M=0, device=device)


def activations(seed: int, M: int, Kin: int, x_type: int, device="cuda"):
    """Device tensor with the values of synth.inputs.activations(seed, M, Kin, x_type)."""
    import torch
    if x_type == BF16:
        x = torch.empty((M, Kin), dtype=torch.int16, device=device)
        fill(K_NORMAL_BF16, seed, 0, x)
    else:
        x = torch.empty((M, Kin), dtype=torch.float32, device=device)
        fill(K_NORMAL_F32, seed, 0, x)
    return x


def moe_hidden(moe, layer: int, device="cuda"):
    """Device copy of synth.inputs.moe_hidden(moe, layer)."""
    from . import inputs
    from .configs import KIND_X
    return activations(gen.tensor_seed(moe.cfg, layer, inputs.MOE_HIDDEN_ID, KIND_X), moe.batch, moe.hidden,
                       F32 if moe.x_type in (F32, I8) else BF16, device)


def moe_inter(moe, layer: int, device="cuda"):
    """Device copy of synth.inputs.moe_inter(moe, layer)."""
    from . import inputs
    from .configs import KIND_X
    return activations(gen.tensor_seed(moe.cfg, layer, inputs.MOE_INTER_ID, KIND_X), moe.batch * moe.top_k,
                       moe.inter, F32 if moe.x_type in (F32, I8) else BF16, device)
