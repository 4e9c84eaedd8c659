"""tq_ternarize against the CPU oracle, bit for bit (trits and scales).

Dense weights are seeded N(0, 0.02^2) fp32 (synth.inputs.dense_weight):
every layout and plane count on small shapes with several group sizes, one
Llama-3.1-8B-shaped projection (4096 x 4096) per layout at full size, the
zero weight, and the codebook check.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle import CODEBOOK, GROUP_F16, TENSOR
from synth import gen, inputs

pytestmark = pytest.mark.gpu
CB = gen.codebook_f16(27)


def _gpu(K, g, layout, w):
    import torch
    from ternary_weight_amd import tq
    N, Kin = w.shape
    d = tq.desc(K, g, layout, N, Kin, n_codebook=27 if layout == CODEBOOK else 0)
    wd = torch.from_numpy(w).cuda()
    trits = torch.full((K, N, Kin), 7, dtype=torch.int8, device="cuda")
    if layout == TENSOR:
        scales = torch.zeros(K, dtype=torch.float32, device="cuda")
    elif layout == GROUP_F16:
        scales = torch.zeros((K, N, Kin // g), dtype=torch.int16, device="cuda")
    else:
        scales = torch.zeros((N, Kin // g), dtype=torch.uint8, device="cuda")
    cb = torch.from_numpy(CB.view(np.int16)).cuda() if layout == CODEBOOK else None
    nws = tq.ternarize_workspace_size(d)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda") if nws else None
    tq.ternarize(d, wd, trits, scales, cb, ws, nws)
    torch.cuda.synchronize()
    s = scales.cpu().numpy()
    return trits.cpu().numpy(), (s.view(np.uint16) if layout == GROUP_F16 else s)


CASES = [(K, g, GROUP_F16) for K in (1, 2, 3, 4) for g in (16, 32, 64, 256)] + \
        [(K, 0, TENSOR) for K in (1, 3)] + [(K, 16, CODEBOOK) for K in (1, 2, 3, 4)] + [(3, 32, CODEBOOK)]


@pytest.mark.parametrize("K,g,layout", CASES, ids=["K%d-g%d-%s" % (K, g, ["tensor", "group", "codebook"][layout])
                                                    for K, g, layout in CASES])
def test_small_shapes_match_oracle(K, g, layout):
    for i, (N, Kin) in enumerate(((37, 256), (64, 512))):
        w = inputs.dense_weight(9, K, 10 * layout + i, N, Kin)
        print("ternarize K=%d g=%d layout=%d %dx%d" % (K, g, layout, N, Kin), flush=True)
        t_ref, s_ref = oracle.ternarize(K, g, layout, w, CB if layout == CODEBOOK else None)
        t, s = _gpu(K, g, layout, w)
        assert np.array_equal(t, t_ref)
        assert np.array_equal(s.view(np.uint8), np.ascontiguousarray(s_ref).view(np.uint8))


@pytest.mark.parametrize("K,g,layout", [(3, 256, GROUP_F16), (1, 0, TENSOR), (3, 16, CODEBOOK)],
                         ids=["group-K3-g256", "tensor-K1", "codebook-d3"])
def test_llama_shaped_projection(K, g, layout):
    w = inputs.dense_weight(9, 0, 100 + layout, 4096, 4096)
    print("ternarize 4096x4096 K=%d g=%d layout=%d" % (K, g, layout), flush=True)
    t_ref, s_ref = oracle.ternarize(K, g, layout, w, CB if layout == CODEBOOK else None)
    t, s = _gpu(K, g, layout, w)
    assert np.array_equal(t, t_ref)
    assert np.array_equal(s.view(np.uint8), np.ascontiguousarray(s_ref).view(np.uint8))


def test_zero_weight_and_codebook_check():
    import torch
    from ternary_weight_amd import tq
    w = np.zeros((16, 64), dtype=np.float32)
    t, s = _gpu(3, 16, GROUP_F16, w)
    assert not t.any() and not s.any()
    t, s = _gpu(2, 0, TENSOR, w)
    assert not t.any() and not s.any()
    d = tq.desc(3, 16, CODEBOOK, 16, 64, n_codebook=27)
    bad = torch.from_numpy(CB[::-1].copy().view(np.int16)).cuda()
    with pytest.raises(tq.TQError) as e:
        tq.ternarize(d, torch.zeros((16, 64), device="cuda"), torch.zeros((3, 16, 64), dtype=torch.int8, device="cuda"),
                     torch.zeros((16, 4), dtype=torch.uint8, device="cuda"), bad)
    assert e.value.status == tq.ERR_VALUE
