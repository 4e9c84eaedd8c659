"""The C ABI without a GPU: the library loads, exports what include/tq.h
declares, and rejects bad arguments before touching the device."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from ternary_weight_amd import tq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tq.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(tq_[a-z0-9_]+)\s*\(", text, re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("tq_pack", "tq_unpack", "tq_gemv", "tq_gemm", "tq_act_quant_int8", "tq_packed_size",
                 "tq_gemv_grouped_prepare", "tq_gemv_grouped_run"):
        assert must in names


def test_library_exports_every_declared_symbol():
    L = tq.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert set(declared_functions()) == set(tq.SIGNATURES)


def test_version_and_status_strings():
    assert tq.abi_version() == 1
    assert tq.status_string(0) == "ok"
    assert tq.status_string(5) == "unsupported combination"


def _status(fn, *args):
    return fn(*args)


def test_descriptor_validation():
    L = tq.lib()
    n = ctypes.c_size_t()
    cases = [
        (tq.desc(0, 64, 1, 64, 64), tq.ERR_ARG),           # no planes
        (tq.desc(5, 64, 1, 64, 64), tq.ERR_ARG),           # too many planes
        (tq.desc(1, 48, 1, 64, 96), tq.ERR_ARG),           # group not a power of two
        (tq.desc(1, 64, 1, 64, 96), tq.ERR_SHAPE),         # Kin % g
        (tq.desc(1, 0, 0, 64, 40), tq.ERR_SHAPE),          # Kin % 16
        (tq.desc(1, 0, 0, -1, 64), tq.ERR_ARG),            # negative
        (tq.desc(1, 0, 7, 64, 64), tq.ERR_ARG),            # bad layout
        (tq.desc(3, 16, 2, 64, 64, n_codebook=0), tq.ERR_ARG),
        (tq.desc(3, 16, 2, 64, 64, n_codebook=33), tq.ERR_ARG),
        (tq.desc(1, 0, 0, 64, 65536 + 16), tq.ERR_SHAPE),
    ]
    for d, want in cases:
        assert L.tq_packed_size(ctypes.byref(d), ctypes.byref(n)) == want, (d.planes, d.group)
        assert tq.last_error() != ""
    assert L.tq_packed_size(ctypes.byref(tq.desc(1, 0, 0, 64, 64)), ctypes.byref(n)) == tq.OK
    assert tq.last_error() == ""


def test_packed_size_accounting():
    # trits: 2 bits each; GROUP_F16: one f16 per plane, row and group
    for K, g in ((1, 256), (2, 256), (3, 256), (4, 256), (2, 64), (2, 32)):
        N, Kin = 4096, 4096
        size = tq.packed_size(tq.desc(K, g, tq.SCALE_GROUP_F16, N, Kin))
        bpw = size * 8 / (N * Kin)
        assert abs(bpw - (2 * K + 16 * K / g)) < 2e-4, (K, g, bpw)
    # per-tensor: 2K bits per weight plus a header and K fp32
    size = tq.packed_size(tq.desc(1, 0, tq.SCALE_TENSOR, 2560, 2560))
    assert size == 256 + 2560 * 2560 // 4 + 256
    # codebook (d = 3, g = 16): 6 bits of trits plus 5-bit indices, six to a dword
    size = tq.packed_size(tq.desc(3, 16, tq.SCALE_CODEBOOK, 4096, 4096, n_codebook=27))
    assert size == 256 + 3 * 4096 * 4096 // 4 + 256 + 4096 * ((256 + 5) // 6) * 4
    # padding rounds rows and columns to 64
    assert tq.packed_size(tq.desc(1, 0, 0, 65, 80)) == 256 + 2 * 2 * 1024 + 256


def test_call_validation_before_any_device_work():
    L = tq.lib()
    d = tq.desc(1, 0, tq.SCALE_TENSOR, 64, 64)
    good = 0x10000
    # misaligned device pointers are refused up front
    assert L.tq_gemv(ctypes.byref(d), good + 4, 1, tq.I8, good, good, good, None, None) == tq.ERR_ALIGN
    assert L.tq_gemv(ctypes.byref(d), good, 17, tq.I8, good, good, good, None, None) == tq.ERR_UNSUPPORTED
    assert L.tq_gemv(ctypes.byref(d), good, -1, tq.I8, good, good, good, None, None) == tq.ERR_ARG
    assert L.tq_gemv(ctypes.byref(d), good, 1, 9, good, good, good, None, None) == tq.ERR_ARG
    assert L.tq_gemv(ctypes.byref(d), None, 1, tq.I8, good, good, good, None, None) == tq.ERR_ARG
    assert L.tq_gemv(ctypes.byref(d), good, 1, tq.I8, good, None, good, None, None) == tq.ERR_ARG
    dg = tq.desc(1, 64, tq.SCALE_GROUP_F16, 64, 64)
    assert L.tq_gemv(ctypes.byref(dg), good, 1, tq.BF16, good, None, good, good, None) == tq.ERR_UNSUPPORTED
    # empty problems are no-ops that need no pointers
    assert L.tq_gemv(ctypes.byref(d), None, 0, tq.I8, None, None, None, None, None) == tq.OK
    d0 = tq.desc(1, 0, tq.SCALE_TENSOR, 0, 64)
    assert L.tq_gemv(ctypes.byref(d0), None, 4, tq.F32, None, None, None, None, None) == tq.OK
    assert L.tq_act_quant_int8(3, 40, tq.F32, good, good, good, None) == tq.ERR_SHAPE
    assert L.tq_act_quant_int8(3, 64, tq.I8, good, good, good, None) == tq.ERR_ARG
    assert L.tq_act_quant_int8(0, 64, tq.F32, None, None, None, None) == tq.OK
    assert L.tq_pack(ctypes.byref(tq.desc(1, 0, 0, 64, 64)), good, good, None, good + 8, None) == tq.ERR_ALIGN
    assert L.tq_pack(ctypes.byref(tq.desc(3, 16, 2, 64, 64, n_codebook=27)), good, good, None, good,
                     None) == tq.ERR_ARG


def test_grouped_validation():
    d1 = tq.desc(1, 0, tq.SCALE_TENSOR, 64, 64)
    d3 = tq.desc(3, 256, tq.SCALE_GROUP_F16, 64, 256)
    good = 0x20000
    probs = tq.problems([(d1, good, good, good, good, None), (d3, good, good, None, good, None)])
    n = tq.gemv_grouped_workspace_size(probs, 1)
    assert n >= 2 * 8
    with pytest.raises(tq.TQError) as e:
        tq.gemv_grouped_prepare(probs, 1, tq.I8, good, n, stream=0)
    assert e.value.status in (tq.ERR_UNSUPPORTED, tq.ERR_ARG)
    with pytest.raises(tq.TQError) as e:
        tq.gemv_grouped_workspace_size(probs, 17)
    assert e.value.status == tq.ERR_UNSUPPORTED
    plan = tq.tq_grouped_plan()
    assert tq.lib().tq_gemv_grouped_run(ctypes.byref(plan), None) == tq.OK   # zero items
    plan.n_items = 5
    plan.workspace = good
    assert tq.lib().tq_gemv_grouped_run(ctypes.byref(plan), None) == tq.ERR_ARG


def test_grouped_tokens_validation():
    """Per-problem token counts: above 16, negative or a NULL list are refused
    before any device call."""
    d1 = tq.desc(1, 0, tq.SCALE_TENSOR, 64, 64)
    good = 0x20000
    probs = tq.problems([(d1, good, good, good, good, None), (d1, good, good, good, good, None)])
    n = tq.gemv_grouped_workspace_size(probs, 16)
    for bad, status in (([17, 1], tq.ERR_UNSUPPORTED), ([1, -1], tq.ERR_ARG)):
        with pytest.raises(tq.TQError) as e:
            tq.gemv_grouped_prepare_tokens(probs, bad, tq.I8, good, n, stream=0)
        assert e.value.status == status
    with pytest.raises(ValueError):
        tq.gemv_grouped_prepare_tokens(probs, [1], tq.I8, good, n, stream=0)
    plan = tq.tq_grouped_plan()
    assert tq.lib().tq_gemv_grouped_prepare_tokens(probs, None, 2, tq.I8, good, n, ctypes.byref(plan),
                                                   None) == tq.ERR_ARG
    d3 = tq.desc(3, 256, tq.SCALE_GROUP_F16, 64, 256)
    mixed = tq.problems([(d1, good, good, good, good, None), (d3, good, good, good, good, None)])
    with pytest.raises(tq.TQError) as e:
        tq.gemv_grouped_prepare_tokens(mixed, [1, 2], tq.I8, good, n, stream=0)
    assert e.value.status == tq.ERR_UNSUPPORTED


def test_gemm_rejects_unsupported_before_device_work():
    L = tq.lib()
    good = 0x30000
    g32 = tq.desc(2, 32, tq.SCALE_GROUP_F16, 64, 64)      # below the int8 MFMA step of 64 columns
    assert L.tq_gemm(ctypes.byref(g32), good, 64, tq.I8, good, good, good, None, None) == tq.ERR_UNSUPPORTED
    cb = tq.desc(3, 16, tq.SCALE_CODEBOOK, 64, 64, n_codebook=27)
    assert L.tq_gemm(ctypes.byref(cb), good, 64, tq.I8, good, good, good, None, None) == tq.ERR_UNSUPPORTED
    d = tq.desc(1, 0, tq.SCALE_TENSOR, 64, 64)
    for xt in (tq.F32, tq.F32_Q8):
        assert L.tq_gemm(ctypes.byref(d), good, 64, xt, good, None, good, None, None) == tq.ERR_UNSUPPORTED
    # x is read 16 bytes at a time; M is bounded; acc only for the bit-exact combination
    assert L.tq_gemm(ctypes.byref(d), good, 64, tq.I8, good + 4, good, good, None, None) == tq.ERR_ALIGN
    assert L.tq_gemm(ctypes.byref(d), good, (1 << 24) + 1, tq.I8, good, good, good, None, None) == tq.ERR_UNSUPPORTED
    assert L.tq_gemm(ctypes.byref(g32), good, 64, tq.BF16, good, None, good, good, None) == tq.ERR_UNSUPPORTED
    assert L.tq_gemm(ctypes.byref(d), None, 0, tq.I8, None, None, None, None, None) == tq.OK


def test_gemm_grouped_validation():
    d1 = tq.desc(1, 0, tq.SCALE_TENSOR, 640, 2560)
    d3 = tq.desc(3, 256, tq.SCALE_GROUP_F16, 640, 2560)
    good = 0x70000
    n = tq.gemm_grouped_workspace_size(tq.problems([(d1, good, good, good, good, None)]), 2048, tq.I8)
    # one item per output tile after the problem table: int8 with one plane
    # and a per-tensor scale takes 128-token x 256-row tiles (16 x 3)
    assert n == 256 + ((16 * 3 * 8 + 255) // 256) * 256
    n3 = tq.gemm_grouped_workspace_size(tq.problems([(d3, good, good, good, good, None)]), 2048, tq.I8)
    # group scales: 128 x 128 tiles (16 x 5)
    assert n3 == 256 + ((16 * 5 * 8 + 255) // 256) * 256
    mixed = tq.problems([(d1, good, good, good, good, None), (d3, good, good, good, good, None)])
    with pytest.raises(tq.TQError) as e:
        tq.gemm_grouped_prepare(mixed, 64, tq.I8, good, 1 << 20, stream=0)
    assert e.value.status == tq.ERR_UNSUPPORTED
    with pytest.raises(tq.TQError) as e:
        tq.gemm_grouped_workspace_size(mixed, 64, tq.F32)
    assert e.value.status == tq.ERR_UNSUPPORTED
    plan = tq.tq_grouped_plan(workspace=good, n_items=3, family=5, n_problems=1)
    assert tq.lib().tq_gemm_grouped_run(ctypes.byref(plan), None) == tq.ERR_ARG   # a decode family
    plan.family = 1000 + 5 * 5 * 4                                                 # past the last family
    assert tq.lib().tq_gemm_grouped_run(ctypes.byref(plan), None) == tq.ERR_ARG
    assert tq.lib().tq_gemv_grouped_run(ctypes.byref(plan), None) == tq.ERR_ARG
    plan.family = 1000 + 2 * 4 + 0                                                 # int8 with groups of 16: none
    assert tq.lib().tq_gemm_grouped_run(ctypes.byref(plan), None) == tq.ERR_ARG


def test_fused_int8_activation_limits():
    L = tq.lib()
    good = 0x40000
    d = tq.desc(1, 0, tq.SCALE_TENSOR, 64, 8192)
    # M * Kin beyond the workgroup's LDS copy
    assert L.tq_gemv(ctypes.byref(d), good, 16, tq.F32_Q8, good, None, good, None, None) == tq.ERR_UNSUPPORTED
    # fp32 activations are read 16 bytes at a time
    assert L.tq_gemv(ctypes.byref(d), good, 1, tq.F32_Q8, good + 4, None, good, None, None) == tq.ERR_ALIGN
    dg = tq.desc(1, 64, tq.SCALE_GROUP_F16, 64, 64)
    assert L.tq_gemv(ctypes.byref(dg), good, 1, tq.F32_Q8, good, None, good, good, None) == tq.ERR_UNSUPPORTED


def test_act_quant_batch_validation():
    L = tq.lib()
    good = 0x50000
    seg = (tq.tq_act_segment * 17)()
    assert L.tq_act_quant_int8_batch(seg, 17, None) == tq.ERR_ARG
    seg[0] = tq.tq_act_segment(2, 40, tq.F32, 0, good, good, good)
    assert L.tq_act_quant_int8_batch(seg, 1, None) == tq.ERR_SHAPE
    seg[0] = tq.tq_act_segment(2, 64, tq.I8, 0, good, good, good)
    assert L.tq_act_quant_int8_batch(seg, 1, None) == tq.ERR_ARG
    seg[0] = tq.tq_act_segment(2, 64, tq.F32, 0, good + 8, good, good)
    assert L.tq_act_quant_int8_batch(seg, 1, None) == tq.ERR_ALIGN
    seg[0] = tq.tq_act_segment(0, 64, tq.F32, 0, None, None, None)
    assert L.tq_act_quant_int8_batch(seg, 1, None) == tq.OK
    assert L.tq_act_quant_int8_batch(None, 0, None) == tq.OK


def test_grouped_run_rejects_forged_plans():
    """A plan not written by prepare: a family out of range (token tiers of 1
    and 4 tokens per pass), a shape above 16 waves, more int8 activations
    than the LDS copy holds, or a per-wave plan that is not one."""
    good = 0x60000
    plan = tq.tq_grouped_plan(workspace=good, n_items=1, family=-1, waves=1, row_blocks=1, n_problems=1)
    fam = lambda xt, layout, K, tier: ((xt * 4 + layout) * 4 + K - 1) * 2 + tier
    for f in (-1, 4 * 16 * 2):
        plan.family = f
        assert tq.lib().tq_gemv_grouped_run(ctypes.byref(plan), None) == tq.ERR_ARG
    plan.family = fam(tq.BF16, 0, 4, 1)      # bf16, per-tensor, 4 planes, 4 tokens
    plan.waves, plan.row_blocks = 16, 2
    assert tq.lib().tq_gemv_grouped_run(ctypes.byref(plan), None) == tq.ERR_ARG
    plan.waves, plan.row_blocks, plan.x_lds_bytes = 1, 1, 65536 + 16
    assert tq.lib().tq_gemv_grouped_run(ctypes.byref(plan), None) == tq.ERR_ARG
    # per-wave items: no such mode, no kernel for the family, items not a whole workgroup
    plan.x_lds_bytes = 0
    plan.mode = 2
    assert tq.lib().tq_gemv_grouped_run(ctypes.byref(plan), None) == tq.ERR_ARG
    plan.mode, plan.row_blocks, plan.n_items = 1, 16, 32
    for f in (fam(tq.F32_Q8, 1, 3, 1), fam(tq.I8, 1, 3, 1), fam(tq.BF16, 2, 3, 1), fam(tq.BF16, 1, 3, 0),
              fam(tq.BF16, 3, 1, 1)):
        plan.family = f
        assert tq.lib().tq_gemv_grouped_run(ctypes.byref(plan), None) == tq.ERR_ARG
    plan.family, plan.n_items = fam(tq.BF16, 1, 3, 1), 24
    assert tq.lib().tq_gemv_grouped_run(ctypes.byref(plan), None) == tq.ERR_ARG

def test_chain_workspace_size_validation():
    """tq_bitnet_chain_workspace_size checks the dimensions on the host."""
    ok = tq.bitnet_dims(2560, 6912, 20, 5, 128, 1e-5)
    n1 = tq.bitnet_chain_workspace_size(ok, 1)
    n30 = tq.bitnet_chain_workspace_size(ok, 30)
    assert n30 > n1 > 0 and n1 % 256 == 0
    bad = [
        (tq.bitnet_dims(2560, 6912, 20, 6, 128, 1e-5), tq.ERR_SHAPE),      # 20 % 6
        (tq.bitnet_dims(2560, 6912, 16, 4, 128, 1e-5), tq.ERR_SHAPE),      # heads * dim != hidden
        (tq.bitnet_dims(2560, 6900, 20, 5, 128, 1e-5), tq.ERR_SHAPE),      # width % 16
        (tq.bitnet_dims(96, 256, 16, 8, 6, 1e-5), tq.ERR_SHAPE),           # head_dim % 4
        (tq.bitnet_dims(20480, 6912, 160, 5, 128, 1e-5), tq.ERR_UNSUPPORTED),   # wider than LDS holds
        (tq.bitnet_dims(2560, 6912, 20, 5, 128, float("nan")), tq.ERR_VALUE),
    ]
    for d, status in bad:
        with pytest.raises(tq.TQError) as e:
            tq.bitnet_chain_workspace_size(d, 1)
        assert e.value.status == status
    with pytest.raises(tq.TQError) as e:
        tq.bitnet_chain_workspace_size(ok, 0)
    assert e.value.status == tq.ERR_ARG


def test_ternarize_workspace_and_validation():
    """tq_ternarize_workspace_size and the host-side checks of tq_ternarize."""
    assert tq.ternarize_workspace_size(tq.desc(3, 256, tq.SCALE_GROUP_F16, 4096, 4096)) == 0
    assert tq.ternarize_workspace_size(tq.desc(1, 0, tq.SCALE_TENSOR, 4096, 4096)) >= 4096 * 16
    with pytest.raises(tq.TQError) as e:
        tq.ternarize_workspace_size(tq.desc(3, 48, tq.SCALE_GROUP_F16, 64, 256))    # 256 % 48
    assert e.value.status in (tq.ERR_SHAPE, tq.ERR_ARG)
    with pytest.raises(tq.TQError) as e:
        tq.ternarize(tq.desc(3, 64, tq.SCALE_GROUP_F16, 64, 256), None, None, None, stream=0)
    assert e.value.status == tq.ERR_ARG
