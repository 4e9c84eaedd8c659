"""Expert-grouped decode (tq_gemv_grouped_prepare_tokens): the routed experts
of mixture-of-experts layers in one launch, each expert with its own token
count, against the oracle run expert by expert.

Inputs come from the seeded generators (synth.inputs / synth.device): a
uniform top-k routing per layer, every expert's gate, up and down fit on
their own (sasori page, "How it works & paper"), the routed tokens' rows
gathered per expert.  The bar is the floating-point paths' per-token relative
error 1e-3 (int8 activations with several planes and group scales included).
"""
from __future__ import annotations

import dataclasses
import gc

import numpy as np
import pytest

import oracle
from oracle import BF16, F32, GROUP_F16
from synth import gen, inputs
from synth.configs import I8, MOES
from tests.gpu_util import TOL, dev, host, pack, rel_err

pytestmark = pytest.mark.gpu


def _run(moe, waves=0, row_blocks=0, fused=False):
    import bench
    import torch
    st = bench.MoeStack(moe, fused=fused)
    st.prepare(waves, row_blocks)
    st.quantize()
    st.gemv()
    torch.cuda.synchronize()
    return st


def _free(st):
    import torch
    del st
    gc.collect()
    torch.cuda.empty_cache()


def _check_all(st):
    import bench
    for (layer, e, p, a, m) in st.meta:
        y = st.ys[layer][p][a:a + m].cpu().numpy()
        ref = bench.moe_reference(st.moe, layer, e, p, a, m)
        err = rel_err(y, ref)
        assert err <= TOL, (layer, e, p, m, err)


def test_moe_small_every_output():
    """Small MoE (2 layers x 16 experts, top-4, 12 tokens, K=3, g=128, bf16 x)."""
    st = _run(MOES["moe_small"])
    assert 4 < st.max_tokens <= 16 and st.plan.family >= 1000    # ~3 tokens each: the matrix cores
    assert len({m for (*_, m) in st.meta}) > 1          # mixed token counts in one launch
    _check_all(st)
    _free(st)


def test_moe_small_split_experts():
    """80 tokens, top-4 of 16: experts hold ~20 tokens and are split into
    problems of 16; a mean count of ~10 puts the plan on the matrix cores."""
    moe = dataclasses.replace(MOES["moe_small"], batch=80)
    st = _run(moe)
    assert st.plan.family >= 1000
    counts = {}
    for (layer, e, p, a, m) in st.meta:
        counts[(layer, e, p)] = counts.get((layer, e, p), 0) + 1
    assert max(counts.values()) > 1
    _check_all(st)
    _free(st)


def test_moe_small_one_token():
    """One token: top-4 experts with one token each, the M = 1 kernels."""
    moe = dataclasses.replace(MOES["moe_small"], batch=1)
    st = _run(moe)
    assert st.max_tokens == 1 and len(st.meta) == 3 * moe.top_k * moe.layers
    _check_all(st)
    _free(st)


@pytest.mark.parametrize("x_type,fused", [(F32, False), (I8, False), (I8, True)])
def test_moe_small_other_activations(x_type, fused):
    """fp32 x; int8 x from the quantiser; fp32 x quantised per token to int8
    inside the product."""
    moe = dataclasses.replace(MOES["moe_small"], x_type=x_type)
    st = _run(moe, fused=fused)
    assert st.quant == (x_type == I8 and not fused)
    _check_all(st)
    _free(st)


@pytest.mark.parametrize("shape", [(4, 1), (1, 4), (2, 2)])
def test_moe_small_plan_shapes(shape):
    """Shapes of the vector-ALU plan (fp32 x: experts of up to 6 tokens in slices of 4)."""
    st = _run(dataclasses.replace(MOES["moe_small"], x_type=F32), *shape)
    assert st.plan.family < 1000 and (st.plan.waves, st.plan.row_blocks) == shape
    _check_all(st)
    _free(st)


@pytest.mark.parametrize("counts", [(3, 0, 1, 16, 5), (9, 0, 16, 8, 12), (1, 0, 2, 6, 1)])
@pytest.mark.parametrize("x_type", [BF16, F32])
def test_tokens_zero_and_mixed(x_type, counts):
    """Problems with mixed token counts in one plan, one of them 0 (NULL
    pointers, no workgroup); f16 group and per-tensor scales.  A mean count
    below 3 keeps bf16 on the vector ALUs (slices of 4, an item per wave),
    3 or more moves it to the matrix cores."""
    import torch
    from ternary_weight_amd import tq
    rng = np.random.default_rng(5)
    for layout, g in ((GROUP_F16, 64), (0, 0)):
        K, N, Kin = 2, 200, 320
        items, refs, outs, tokens = [], [], [], []
        keep = []
        for i, m in enumerate(counts):
            trits = rng.integers(-1, 2, size=(K, N, Kin)).astype(np.int8)
            if layout == GROUP_F16:
                scales = gen.f16_bits(rng.uniform(0.01, 0.1, size=(K, N, Kin // g)))
            else:
                scales = rng.uniform(0.01, 0.1, size=K).astype(np.float32)
            d, blob = pack(K, g, layout, trits, scales)
            keep.append((d, blob))
            if m == 0:
                items.append((d, blob, None, None, None, None))
                refs.append(None)
                outs.append(None)
            else:
                x = inputs.activations(1000 + i, m, Kin, x_type)
                y = torch.full((m, N), float("nan"), dtype=torch.float32, device="cuda")
                items.append((d, blob, dev(x), None, y, None))
                refs.append(oracle.gemv_fp(K, g, layout, trits, scales, x, x_type, None))
                outs.append(y)
                keep.append(x)
            tokens.append(m)
        probs = tq.problems(items)
        ws = torch.empty(tq.gemv_grouped_workspace_size(probs, 16), dtype=torch.uint8, device="cuda")
        plan = tq.gemv_grouped_prepare_tokens(probs, tokens, x_type, ws, ws.numel())
        mfma = x_type == BF16 and sum(counts) >= 3 * sum(c > 0 for c in counts)
        assert (plan.family >= 1000) == mfma and plan.M == max(counts)
        if not mfma:   # one expert has more tokens than a pass: slices
            assert plan.mode == (1 if x_type == BF16 else 0)
        tq.gemv_grouped_run(plan)
        torch.cuda.synchronize()
        for y, ref in zip(outs, refs):
            if y is not None:
                assert rel_err(host(y), ref) <= TOL


def test_moe_full_size_sampled():
    """Qwen3-30B-A3B expert shapes, 48 layers x 128 experts, 64 tokens, in the
    benchmark's launch: sampled rows of the first, last and three other
    problems against the oracle."""
    import bench
    st = _run(MOES["moe"])
    rng = np.random.default_rng(7)
    picks = sorted({0, len(st.meta) - 1, *rng.integers(len(st.meta), size=3).tolist()})
    for i in picks:
        layer, e, p, a, m = st.meta[i]
        n = st.shapes[p][1]
        r = np.sort(rng.choice(n, size=32, replace=False))
        y = st.ys[layer][p][a:a + m].cpu().numpy()[:, r]
        err = rel_err(y, bench.moe_reference(st.moe, layer, e, p, a, m, rows=r))
        assert err <= TOL, (layer, e, p, m, err)
    _free(st)
