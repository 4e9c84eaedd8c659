"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (bench.Stack: every projection of the stack packed in one
slab, one grouped launch per step), on outputs the oracle computes one by one.

Each stack is generated on the GPU by the device copy of the seeded
generator; the oracle regenerates the sampled rows (and their activations)
on the host from the same counters, so no input crosses from the GPU side.
Samples: the first and last projection of the stack and one in between,
64 random rows each for every token; for the one-token decode stacks also
every projection of every layer, 8 random rows each; for the prefill stacks
also every row of one projection for 16 random tokens.  Bars: bit-exact for int8
activations with one plane and a per-tensor scale, else the per-token
relative error 1e-3.
"""
from __future__ import annotations

import gc

import numpy as np
import pytest

import oracle
from oracle import BF16, F32, I8
from synth import inputs
from synth.configs import CASES, TENSOR
from tests.gpu_util import TOL, rel_err

pytestmark = pytest.mark.gpu


def _stack(name, M=None, fused=False):
    import bench
    case = CASES[name]
    st = bench.Stack(case, case.M if M is None else M, fused=fused)
    st.prepare()
    st.quantize()
    st.gemv()
    import torch
    torch.cuda.synchronize()
    return st


def _free(st):
    import torch
    del st
    gc.collect()
    torch.cuda.empty_cache()


def _reference(case, h, x_type):
    if x_type == I8:
        q, s = oracle.act_quant_i8(h["x"], F32)
        return oracle.gemv_i8(case.planes, case.group, case.layout, h["trits"], h["scales"], q, s, h["codebook"])
    return oracle.gemv_fp(case.planes, case.group, case.layout, h["trits"], h["scales"], h["x"], x_type,
                          h["codebook"])


def _check_rows(st, seed, rows=64):
    case, M = st.case, st.M
    rng = np.random.default_rng(seed)
    picks = sorted({0, len(st.projs) - 1, int(rng.integers(1, len(st.projs) - 1))})
    exact = case.x_type == I8 and case.layout == TENSOR and case.planes == 1
    for i in picks:
        layer, p, name, n, kin = st.projs[i]
        r = np.sort(rng.choice(n, size=min(rows, n), replace=False))
        h = inputs.projection(case, layer, p, n, kin, rows=r, M=M)
        y = st.ys[i].detach().cpu().numpy()[:, r]
        ref = _reference(case, h, case.x_type)
        if exact:
            assert np.array_equal(y.view(np.uint32), ref["y32"].view(np.uint32)), (name, layer)
        else:
            ystar = ref["y64"] if case.x_type == I8 else ref
            err = rel_err(y, ystar)
            assert err <= TOL, (name, layer, err)


def _check_every_projection(st, seed, rows=8):
    """Every projection of every layer: `rows` random rows for every token."""
    case, M = st.case, st.M
    rng = np.random.default_rng(seed)
    exact = case.x_type == I8 and case.layout == TENSOR and case.planes == 1
    ys = [y.detach().cpu().numpy() for y in st.ys]
    for i, (layer, p, name, n, kin) in enumerate(st.projs):
        r = np.sort(rng.choice(n, size=min(rows, n), replace=False))
        h = inputs.projection(case, layer, p, n, kin, rows=r, M=M)
        ref = _reference(case, h, case.x_type)
        y = ys[i][:, r]
        if exact:
            assert np.array_equal(y.view(np.uint32), ref["y32"].view(np.uint32)), (name, layer)
        else:
            err = rel_err(y, ref["y64"] if case.x_type == I8 else ref)
            assert err <= TOL, (name, layer, err)


def test_tiny_linear_full():
    """256 x 512, one plane, f16 scale per group of 64, fp32 x: every output."""
    from ternary_weight_amd import tq
    import torch
    case = CASES["cfg1"]
    (_, _, _, n, kin), = case.projections()
    from synth import device
    d = device.projection(case, 0, 0, n, kin)
    desc = tq.desc(1, 64, case.layout, n, kin)
    blob = torch.empty(tq.packed_size(desc), dtype=torch.uint8, device="cuda")
    tq.pack(desc, d["trits"], d["scales"], None, blob)
    y = torch.empty((1, n), dtype=torch.float32, device="cuda")
    tq.gemv(desc, blob, 1, F32, d["x"], None, y)
    torch.cuda.synchronize()
    h = inputs.projection(case, 0, 0, n, kin)
    ref = oracle.gemv_fp(1, 64, case.layout, h["trits"], h["scales"], h["x"], F32)
    assert rel_err(y.cpu().numpy(), ref) <= 1e-5


def test_bitnet_decode_stack():
    st = _stack("cfg2")
    _check_rows(st, 2)
    _check_every_projection(st, 12)
    # the fused launch (quantisation inside the product) gives the same bits
    import torch
    ys = [y.clone() for y in st.ys]
    _free(st)
    st2 = _stack("cfg2", fused=True)
    for a, b in zip(ys, st2.ys):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    _free(st2)


def test_llama_shaped_k3_decode_stack():
    st = _stack("cfg3")
    _check_rows(st, 3)
    _check_every_projection(st, 13)
    _free(st)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_codec_d3_decode_stack(M):
    st = _stack("cfg4", M=M)
    _check_rows(st, 40 + M)
    if M == 1:
        _check_every_projection(st, 14)
    _free(st)


@pytest.mark.parametrize("name", ["cfg5a", "cfg5b"])
def test_prefill_stack(name):
    st = _stack(name)
    _check_rows(st, 5)
    # every row of one projection for 16 random tokens
    case, M = st.case, st.M
    rng = np.random.default_rng(55)
    i = int(rng.integers(len(st.projs)))
    layer, p, pname, n, kin = st.projs[i]
    toks = np.sort(rng.choice(M, size=16, replace=False))
    h = inputs.projection(case, layer, p, n, kin, M=M)
    h["x"] = h["x"][toks]
    y = st.ys[i].detach().cpu().numpy()[toks]
    ref = _reference(case, h, case.x_type)
    if case.x_type == I8:
        assert np.array_equal(y.view(np.uint32), ref["y32"].view(np.uint32)), pname
    else:
        assert rel_err(y, ref) <= TOL
    _free(st)
