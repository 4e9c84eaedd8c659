"""tq_ternarize_noalloc (the entry point that allocates nothing) against
tq_ternarize (the same fit with a caller-owned workspace), bit for bit,
through the C ABI: two calls in a row on the library's scratch array, the
second with fewer rows, then the row limit and the layouts that need no
scratch."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import CODEBOOK, GROUP_F16, TENSOR
from synth import gen, inputs

pytestmark = pytest.mark.gpu
CB = gen.codebook_f16(27)


def _outputs(K, g, layout, N, Kin):
    import torch
    trits = torch.full((K, N, Kin), 7, dtype=torch.int8, device="cuda")
    if layout == TENSOR:
        scales = torch.full((K,), float("nan"), dtype=torch.float32, device="cuda")
    elif layout == GROUP_F16:
        scales = torch.zeros((K, N, Kin // g), dtype=torch.int16, device="cuda")
    else:
        scales = torch.zeros((N, Kin // g), dtype=torch.uint8, device="cuda")
    return trits, scales


def _both(K, g, layout, w):
    """(trits, scales) from tq_ternarize with a workspace and from tq_ternarize_noalloc."""
    import torch
    from ternary_weight_amd import tq
    N, Kin = w.shape
    d = tq.desc(K, g, layout, N, Kin, n_codebook=27 if layout == CODEBOOK else 0)
    wd = torch.from_numpy(w).cuda()
    cb = torch.from_numpy(CB.view(np.int16)).cuda() if layout == CODEBOOK else None
    t1, s1 = _outputs(K, g, layout, N, Kin)
    nws = tq.ternarize_workspace_size(d)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda") if nws else None
    tq.ternarize(d, wd, t1, s1, cb, ws, nws)
    t2, s2 = _outputs(K, g, layout, N, Kin)
    tq.ternarize_noalloc(d, wd, t2, s2, cb)
    torch.cuda.synchronize()
    return (t1.cpu().numpy(), s1.cpu().numpy()), (t2.cpu().numpy(), s2.cpu().numpy())


def _same(a, b):
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(np.ascontiguousarray(a[1]).view(np.uint8), np.ascontiguousarray(b[1]).view(np.uint8))


def test_noalloc_tensor_two_calls_second_smaller():
    # a first call over many rows leaves its sums in the scratch array; the
    # second, smaller one must not pick any of them up
    for i, (N, Kin) in enumerate(((3000, 1024), (700, 512))):
        w = inputs.dense_weight(11, i, 7, N, Kin)
        print("noalloc tensor K=3 %d x %d" % (N, Kin), flush=True)
        ref, got = _both(3, 0, TENSOR, w)
        _same(ref, got)
        assert np.all(np.isfinite(got[1])) and np.all(np.abs(got[0]) <= 1)


def test_noalloc_row_limit_and_other_layouts():
    import torch
    from ternary_weight_amd import tq
    lim = 1 << 18
    w = inputs.dense_weight(11, 3, 8, lim, 16)
    print("noalloc tensor K=1 %d x 16 (the row limit)" % lim, flush=True)
    ref, got = _both(1, 0, TENSOR, w)
    _same(ref, got)
    d = tq.desc(1, 0, TENSOR, lim + 1, 16)
    t, s = _outputs(1, 0, TENSOR, 1, 16)
    with pytest.raises(tq.TQError) as e:
        tq.ternarize_noalloc(d, torch.zeros(16, device="cuda"), t, s)
    assert e.value.status == tq.ERR_UNSUPPORTED
    for K, g, layout in ((3, 64, GROUP_F16), (3, 16, CODEBOOK)):
        w = inputs.dense_weight(11, 4, 9 + layout, 96, 256)
        ref, got = _both(K, g, layout, w)
        _same(ref, got)
