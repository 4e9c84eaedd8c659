"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (bench.Stack: every projection of the stack packed in one
slab, one grouped launch per step).

Coverage:
  - the one-token decode stacks (BitNet-2B int8, Llama-8B-shaped K=3 g=256,
    the d=3 codec): every output of every projection of every layer;
  - the codec at 4 and 16 tokens: every output of the first and the last
    layer for every token, and 64 random rows of a few other projections;
  - the codec packed with compact base-3 codes: the same, every output at
    one token;
  - the BitNet-2B prefill stack (2048 tokens, int8): every output of the
    first and the last layer; every other layer sampled (16 random tokens x
    every row, and every token x 16 random rows, for every projection);
  - the Llama-8B-shaped prefill stack (512 tokens, K=3): for every
    projection of the first and the last layer, 64 random tokens x every row
    and every token x 64 random rows; every other layer sampled (2 random
    tokens x every row, every token x 8 random rows).

Each stack is generated on the GPU by the device copy of the seeded input
generator.  The oracle takes the canonical arrays of each projection from
that same generator -- drawn again on the device and copied to the host,
since the host copy of the generator is too slow for billions of weights
(test_gpu_synth shows the two copies equal bit for bit) -- and never sees a
packed blob or a product output.  Bars: bit-exact for int8 activations
with one plane and a per-tensor scale, else the per-token relative error
1e-3.
"""
from __future__ import annotations

import gc

import numpy as np
import pytest

import oracle
from oracle import BF16, F32, I8
from synth import inputs
from synth.configs import CASES, CODEBOOK, GROUP_F16, TENSOR
from tests.gpu_util import TOL, rel_err

pytestmark = pytest.mark.gpu


def _stack(name, M=None, fused=False, b3=False):
    import bench
    import torch
    case = CASES[name]
    st = bench.Stack(case, case.M if M is None else M, fused=fused, b3=b3)
    st.prepare()
    st.quantize()
    st.gemv()
    torch.cuda.synchronize()
    return st


def _free(st=None):
    import torch
    del st
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _canonical(case, layer, p, n, kin, M):
    """Host copies of the canonical arrays of one projection (device generator)."""
    from synth import device
    d = device.projection(case, layer, p, n, kin, M=M)
    h = {"trits": d["trits"].cpu().numpy()}
    if case.layout == GROUP_F16:
        h["scales"] = d["scales"].cpu().numpy().view(np.uint16)
    elif case.layout == CODEBOOK:
        h["scales"] = d["scales"].cpu().numpy()
    else:
        h["scales"] = d["scales"].cpu().numpy()
    h["codebook"] = None if d["codebook"] is None else d["codebook"].cpu().numpy().view(np.uint16)
    x = d["x"].cpu().numpy()
    h["x"] = x.view(np.uint16) if case.x_type == BF16 else x
    del d
    return h


def _restrict(case, h, rows=None, toks=None):
    """The arrays of a subset of output rows and tokens."""
    out = dict(h)
    if rows is not None:
        out["trits"] = np.ascontiguousarray(h["trits"][:, rows, :])
        if case.layout == GROUP_F16:
            out["scales"] = np.ascontiguousarray(h["scales"][:, rows, :])
        elif case.layout == CODEBOOK:
            out["scales"] = np.ascontiguousarray(h["scales"][rows])
    if toks is not None:
        out["x"] = np.ascontiguousarray(h["x"][toks])
    return out


def _reference(case, h):
    if case.x_type == I8:
        q, s = oracle.act_quant_i8(h["x"], F32)
        return oracle.gemv_i8(case.planes, case.group, case.layout, h["trits"], h["scales"], q, s, h["codebook"])
    return oracle.gemv_fp(case.planes, case.group, case.layout, h["trits"], h["scales"], h["x"], case.x_type,
                          h["codebook"])


def _exact(case):
    return case.x_type == I8 and case.layout == TENSOR and case.planes == 1


def _compare(case, y, ref, what):
    """y fp32 [tokens][rows] against the oracle's result for the same outputs."""
    if _exact(case):
        assert np.array_equal(y.view(np.uint32), ref["y32"].view(np.uint32)), what
        return 0.0
    err = rel_err(y, ref["y64"] if case.x_type == I8 else ref)
    assert err <= TOL, (what, err)
    return err


def _check_projection(st, i, rows=None, toks=None, h=None):
    """Outputs (rows x toks; None = all) of projection i of the stack."""
    case, M = st.case, st.M
    layer, p, name, n, kin = st.projs[i]
    if h is None:
        h = _canonical(case, layer, p, n, kin, M)
    ref = _reference(case, _restrict(case, h, rows, toks))
    y = st.ys[i].detach().cpu().numpy()
    if toks is not None:
        y = y[toks]
    if rows is not None:
        y = y[:, rows]
    return _compare(case, np.ascontiguousarray(y), ref, (name, layer, "rows", None if rows is None else len(rows),
                                                         "tokens", None if toks is None else len(toks)))


def _check_every_output(st, idxs):
    worst = 0.0
    for i in idxs:
        worst = max(worst, _check_projection(st, i))
    return worst


def _layer_projs(st, layer):
    return [i for i, pr in enumerate(st.projs) if pr[0] == layer]


def _check_sampled_rows(st, seed, rows=64, idxs=None):
    """64 random rows of some projections for every token, the oracle on the
    host copy of the generator (an independent route to the inputs)."""
    case, M = st.case, st.M
    rng = np.random.default_rng(seed)
    if idxs is None:
        idxs = sorted({0, len(st.projs) - 1, int(rng.integers(1, len(st.projs) - 1))})
    for i in idxs:
        layer, p, name, n, kin = st.projs[i]
        r = np.sort(rng.choice(n, size=min(rows, n), replace=False))
        h = inputs.projection(case, layer, p, n, kin, rows=r, M=M)
        y = np.ascontiguousarray(st.ys[i].detach().cpu().numpy()[:, r])
        _compare(case, y, _reference(case, h), (name, layer, "host-generated rows"))


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


def test_bitnet_decode_stack_every_output():
    """BitNet-2B, 30 layers x 7 projections, int8: all 210 GEMVs bit for bit,
    with the separate quantiser and with quantisation inside the product."""
    import torch
    print("cfg2 M=1: every output of 210 projections", flush=True)
    st = _stack("cfg2")
    _check_sampled_rows(st, 2)
    _check_every_output(st, range(len(st.projs)))
    ys = [y.clone() for y in st.ys]
    _free(st)
    st2 = _stack("cfg2", fused=True)
    for a, b in zip(ys, st2.ys):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    _free(st2)


@pytest.mark.parametrize("name", ["cfg3", "cfg4"])
def test_llama_shaped_decode_stack_every_output(name):
    """Llama-8B shapes, 32 layers x 7 projections, one token: all 224 GEMVs."""
    print("%s M=1: every output of 224 projections" % name, flush=True)
    st = _stack(name)
    _check_sampled_rows(st, 3)
    worst = _check_every_output(st, range(len(st.projs)))
    print("%s worst per-token relative error %.3g" % (name, worst), flush=True)
    _free(st)


@pytest.mark.parametrize("M", [4, 16])
def test_codec_several_tokens(M):
    """The codec at 4 and 16 tokens: first and last layer in full."""
    print("cfg4 M=%d: first and last layer in full" % M, flush=True)
    st = _stack("cfg4", M=M)
    _check_sampled_rows(st, 40 + M)
    last = st.case.model["layers"] - 1
    worst = _check_every_output(st, _layer_projs(st, 0) + _layer_projs(st, last))
    print("cfg4 M=%d worst per-token relative error %.3g" % (M, worst), flush=True)
    _free(st)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_codec_compact_codes(M):
    """The codec stack packed with compact base-3 codes (same canonical arrays,
    the same oracle): every output at one token, the first and last layer in
    full at 4 and 16 tokens."""
    print("cfg4 compact codes M=%d" % M, flush=True)
    st = _stack("cfg4", M=M, b3=True)
    _check_sampled_rows(st, 80 + M)
    last = st.case.model["layers"] - 1
    idxs = range(len(st.projs)) if M == 1 else _layer_projs(st, 0) + _layer_projs(st, last)
    worst = _check_every_output(st, idxs)
    print("cfg4 compact codes M=%d worst per-token relative error %.3g" % (M, worst), flush=True)
    _free(st)


@pytest.fixture(scope="module")
def prefill_i8():
    print("cfg5a: building the stack (M=2048)", flush=True)
    st = _stack("cfg5a")
    yield st
    _free(st)


@pytest.mark.parametrize("which", ["first", "last"])
def test_bitnet_prefill_layer_in_full(prefill_i8, which):
    """BitNet-2B prefill, 2048 tokens, int8: every output of the layer, bit for bit."""
    st = prefill_i8
    layer = 0 if which == "first" else st.case.model["layers"] - 1
    print("cfg5a: every output of layer %d" % layer, flush=True)
    _check_every_output(st, _layer_projs(st, layer))


def test_bitnet_prefill_other_layers_sampled(prefill_i8):
    st = prefill_i8
    rng = np.random.default_rng(51)
    last = st.case.model["layers"] - 1
    print("cfg5a: layers 1..%d sampled" % (last - 1), flush=True)
    for i, (layer, p, name, n, kin) in enumerate(st.projs):
        if layer in (0, last):
            continue
        h = _canonical(st.case, layer, p, n, kin, st.M)
        toks = np.sort(rng.choice(st.M, size=16, replace=False))
        rows = np.sort(rng.choice(n, size=16, replace=False))
        _check_projection(st, i, toks=toks, h=h)
        _check_projection(st, i, rows=rows, h=h)


@pytest.fixture(scope="module")
def prefill_bf16():
    print("cfg5b: building the stack (M=512)", flush=True)
    st = _stack("cfg5b")
    yield st
    _free(st)


@pytest.mark.parametrize("which", ["first", "last"])
def test_llama_prefill_layer(prefill_bf16, which):
    """Llama-8B-shaped prefill, 512 tokens, K=3: every projection of the
    layer, 64 random tokens x every row and every token x 64 random rows."""
    st = prefill_bf16
    layer = 0 if which == "first" else st.case.model["layers"] - 1
    rng = np.random.default_rng(61 + layer)
    print("cfg5b: layer %d, 64 tokens x all rows and all tokens x 64 rows" % layer, flush=True)
    worst = 0.0
    for i in _layer_projs(st, layer):
        _, p, name, n, kin = st.projs[i]
        h = _canonical(st.case, layer, p, n, kin, st.M)
        toks = np.sort(rng.choice(st.M, size=64, replace=False))
        rows = np.sort(rng.choice(n, size=64, replace=False))
        worst = max(worst, _check_projection(st, i, toks=toks, h=h), _check_projection(st, i, rows=rows, h=h))
    print("cfg5b layer %d worst per-token relative error %.3g" % (layer, worst), flush=True)


def test_llama_prefill_other_layers_sampled(prefill_bf16):
    st = prefill_bf16
    rng = np.random.default_rng(71)
    last = st.case.model["layers"] - 1
    _check_sampled_rows(st, 5)
    print("cfg5b: layers 1..%d sampled" % (last - 1), flush=True)
    for i, (layer, p, name, n, kin) in enumerate(st.projs):
        if layer in (0, last):
            continue
        h = _canonical(st.case, layer, p, n, kin, st.M)
        toks = np.sort(rng.choice(st.M, size=2, replace=False))
        rows = np.sort(rng.choice(n, size=8, replace=False))
        _check_projection(st, i, toks=toks, h=h)
        _check_projection(st, i, rows=rows, h=h)
