"""GPU parity of the HIP library against the CPU oracle, through the C ABI.

Bars: bit-exact for packing, the int8 quantiser and the int8-activation
per-tensor path (y and the int32 accumulator); per-token relative error
max_n |y - y*| / max(|y*|, rms(y*)) <= 1e-3 against the fp64 oracle for the
floating-point paths.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle import BF16, CODEBOOK, F32, GROUP_F16, I8, TENSOR

F32_Q8 = 3   # fp32 activations quantised to int8 inside the product
from synth import gen

from tests.gpu_util import TOL, dev, gemv, host, pack, read_blob, rel_err, torch

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(1234)


def rand_problem(K, g, layout, N, Kin, rng=RNG, p=(0.3, 0.4, 0.3)):
    trits = rng.choice(np.array([-1, 0, 1], dtype=np.int8), size=(K, N, Kin), p=list(p))
    cb = None
    if layout == TENSOR:
        scales = (10 ** rng.uniform(-3, -1, size=K)).astype(np.float32)
    elif layout == GROUP_F16:
        scales = gen.f16_bits(10 ** rng.uniform(-3, -1, size=(K, N, Kin // g)) / 3.0 ** np.arange(K)[:, None, None])
    else:
        scales = rng.integers(0, 27, size=(N, Kin // g), dtype=np.uint8)
        cb = gen.codebook_f16(27)
    return trits, scales, cb


def rand_x(M, Kin, x_type, rng=RNG):
    v = rng.standard_normal((M, Kin))
    return gen.bf16_bits(v) if x_type == BF16 else v.astype(np.float32)


# ---------------------------------------------------------------------------
# Packing.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("K,g,layout,N,Kin", [
    (1, 0, TENSOR, 64, 64), (1, 0, TENSOR, 100, 48), (3, 256, GROUP_F16, 130, 512),
    (2, 16, GROUP_F16, 64, 80), (4, 32, GROUP_F16, 7, 96), (3, 16, CODEBOOK, 65, 208),
    (1, 64, GROUP_F16, 256, 512), (3, 128, GROUP_F16, 1, 384),
])
def test_pack_layout_and_roundtrip(K, g, layout, N, Kin):
    from ternary_weight_amd import tq
    t = torch()
    trits, scales, cb = rand_problem(K, g, layout, N, Kin)
    d, blob = pack(K, g, layout, trits, scales, cb)
    raw = host(blob)
    got = read_blob(raw, K, N, Kin, layout, g)
    assert np.array_equal(got["trits"], trits)
    assert not np.any(got["codes"] == 3)                      # code 11 never written
    pad = got["codes"].copy()
    pad[:, :N, :Kin] = 0
    assert not np.any(pad)                                     # padding is code 00
    assert np.array_equal(got["scales"], scales)
    if layout == CODEBOOK:
        assert np.array_equal(got["codebook"][:27], cb) and not np.any(got["codebook"][27:])
    hdr = raw[:256].view(np.uint32)
    assert hdr[0] == 0x31575154 and hdr[16] == 0              # magic, pack status
    # unpack gives the canonical arrays back
    tr2 = t.zeros((K, N, Kin), dtype=t.int8, device="cuda")
    sc2 = t.zeros_like(dev(scales))
    cb2 = t.zeros(27, dtype=t.int16, device="cuda") if cb is not None else None
    tq.unpack(d, blob, tr2, sc2, cb2)
    t.cuda.synchronize()
    assert np.array_equal(host(tr2), trits)
    assert np.array_equal(host(sc2).view(scales.dtype), scales)
    if cb is not None:
        assert np.array_equal(host(cb2, np.uint16), cb)


def test_pack_all_81_byte_patterns():
    # every combination of four trits appears in some byte
    combos = np.array(np.meshgrid(*[[-1, 0, 1]] * 4, indexing="ij")).reshape(4, -1).T   # [81][4]
    Kin = 16 * 96
    row = np.zeros(Kin, dtype=np.int8)
    # place the four trits of a combination in the four columns that share a byte:
    # columns 16d + 4p + b for p = 0..3 share byte b of dword d
    for i, c in enumerate(combos):
        d, b = divmod(i, 4)
        for p in range(4):
            row[16 * d + 4 * p + b] = c[p]
    trits = np.stack([row, -row, np.roll(row, 16)])[None].repeat(1, 0).reshape(1, 3, Kin)
    scales = np.array([0.5], dtype=np.float32)
    d, blob = pack(1, 0, TENSOR, trits, scales)
    got = read_blob(host(blob), 1, 3, Kin, TENSOR)
    assert np.array_equal(got["trits"], trits)
    by = host(blob)[256:256 + 3 * 1024 * 2].reshape(-1)
    assert len(set(by[:81 // 4 * 4].tolist())) > 16


def test_pack_rejects_bad_values():
    from ternary_weight_amd import tq
    trits, scales, _ = rand_problem(1, 64, GROUP_F16, 64, 128)
    bad = trits.copy()
    bad[0, 5, 7] = 2
    with pytest.raises(tq.TQError) as e:
        pack(1, 64, GROUP_F16, bad, scales)
    assert e.value.status == tq.ERR_VALUE
    s2 = scales.copy()
    s2[0, 3, 1] = 0x7C00                                       # f16 infinity
    with pytest.raises(tq.TQError) as e:
        pack(1, 64, GROUP_F16, trits, s2)
    assert e.value.status == tq.ERR_VALUE
    t3, idx, cb = rand_problem(3, 16, CODEBOOK, 64, 64)
    idx = idx.copy()
    idx[2, 1] = 27
    with pytest.raises(tq.TQError) as e:
        pack(3, 16, CODEBOOK, t3, idx, cb)
    assert e.value.status == tq.ERR_VALUE


# ---------------------------------------------------------------------------
# int8 quantiser.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("x_type", [F32, BF16])
@pytest.mark.parametrize("M,Kin", [(1, 2560), (5, 6912), (3, 16), (64, 4096)])
def test_act_quant_bit_exact(x_type, M, Kin):
    from ternary_weight_amd import tq
    t = torch()
    v = RNG.standard_normal((M, Kin)) * 10.0 ** RNG.uniform(-20, 20, size=(M, 1))
    if M > 2:
        v[1] = 0.0
        v[2, : Kin // 2] = 0.0
    x = gen.bf16_bits(v) if x_type == BF16 else v.astype(np.float32)
    qd = t.empty((M, Kin), dtype=t.int8, device="cuda")
    sd = t.empty(M, dtype=t.float32, device="cuda")
    tq.act_quant_int8(M, Kin, x_type, dev(x), qd, sd)
    t.cuda.synchronize()
    q, s = oracle.act_quant_i8(x, x_type)
    assert np.array_equal(host(qd), q)
    assert np.array_equal(host(sd).view(np.uint32), s.view(np.uint32))


# ---------------------------------------------------------------------------
# Decode products.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("N,Kin,M", [(64, 64, 1), (2560, 2560, 1), (640, 2560, 1), (100, 6912, 1),
                                     (96, 80, 3), (200, 1040, 4), (130, 512, 7), (64, 256, 16),
                                     # 8 tokens and more: the wide kernels, 512 rows a workgroup
                                     (640, 2560, 8), (1000, 1040, 12), (2560, 2560, 16), (513, 512, 9)])
def test_gemv_int8_per_tensor_bit_exact(N, Kin, M):
    trits, scales, _ = rand_problem(1, 0, TENSOR, N, Kin)
    x = rand_x(M, Kin, F32)
    q, s = oracle.act_quant_i8(x)
    d, blob = pack(1, 0, TENSOR, trits, scales)
    y, acc = gemv(d, blob, I8, q, s, want_acc=True)
    ref = oracle.gemv_i8(1, 0, TENSOR, trits, scales, q, s)
    assert np.array_equal(acc, ref["acc"].astype(np.int32))
    assert np.array_equal(y.view(np.uint32), ref["y32"].view(np.uint32))


FP_CASES = []
for layout in (TENSOR, GROUP_F16, CODEBOOK):
    for K in (1, 2, 3, 4):
        for g in ((0,) if layout == TENSOR else (16, 32, 64, 128, 256)):
            if layout == CODEBOOK and (K != 3 and g != 16):
                continue
            FP_CASES.append((layout, K, g))


@pytest.mark.parametrize("layout,K,g", FP_CASES)
@pytest.mark.parametrize("x_type", [F32, BF16, I8, F32_Q8])
def test_gemv_all_formats(layout, K, g, x_type):
    rng = np.random.default_rng(K * 1000 + g + 7 * layout + 31 * x_type)
    N, Kin = 192, 1024 + (256 if g <= 256 else 0)
    for M in (1, 3, 4, 16):
        trits, scales, cb = rand_problem(K, g, layout, N, Kin, rng)
        d, blob = pack(K, g, layout, trits, scales, cb)
        if x_type in (I8, F32_Q8):
            xf = rand_x(M, Kin, F32, rng)
            q, s = oracle.act_quant_i8(xf)
            y = gemv(d, blob, I8, q, s) if x_type == I8 else gemv(d, blob, F32_Q8, xf)
            ref = oracle.gemv_i8(K, g, layout, trits, scales, q, s, cb)
            if layout == TENSOR and K == 1:
                assert np.array_equal(y.view(np.uint32), ref["y32"].view(np.uint32))
            else:
                assert rel_err(y, ref["y64"]) <= TOL
        else:
            x = rand_x(M, Kin, x_type, rng)
            y = gemv(d, blob, x_type, x)
            ref = oracle.gemv_fp(K, g, layout, trits, scales, x, x_type, cb)
            err = rel_err(y, ref)
            assert err <= TOL, (M, err)
            assert err <= 1e-5          # fp32 accumulation is far inside the bar


def test_gemv_ragged_and_edge_shapes():
    for (K, g, layout, N, Kin, M, xt) in [
        (1, 0, TENSOR, 1, 16, 1, I8), (1, 0, TENSOR, 65, 48, 2, I8), (3, 16, CODEBOOK, 3, 48, 5, BF16),
        (2, 16, GROUP_F16, 63, 80, 1, BF16), (3, 256, GROUP_F16, 129, 768, 1, BF16),
        (1, 64, GROUP_F16, 1, 960, 16, F32), (4, 32, GROUP_F16, 200, 32, 4, BF16),
        (1, 0, TENSOR, 64, 65536, 1, I8),
    ]:
        trits, scales, cb = rand_problem(K, g, layout, N, Kin)
        d, blob = pack(K, g, layout, trits, scales, cb)
        if xt == I8:
            q, s = oracle.act_quant_i8(rand_x(M, Kin, F32))
            y = gemv(d, blob, I8, q, s)
            ref = oracle.gemv_i8(K, g, layout, trits, scales, q, s, cb)
            if layout == TENSOR and K == 1:
                assert np.array_equal(y.view(np.uint32), ref["y32"].view(np.uint32))
            else:
                assert rel_err(y, ref["y64"]) <= TOL
        else:
            x = rand_x(M, Kin, xt)
            y = gemv(d, blob, xt, x)
            assert rel_err(y, oracle.gemv_fp(K, g, layout, trits, scales, x, xt, cb)) <= TOL


def test_gemv_zero_in_features_gives_zeros():
    from ternary_weight_amd import tq
    t = torch()
    d = tq.desc(1, 0, tq.SCALE_TENSOR, 70, 0)
    blob = t.zeros(tq.packed_size(d), dtype=t.uint8, device="cuda")
    tq.pack(d, None, dev(np.array([0.5], np.float32)), None, blob)
    y, acc = gemv(d, blob, I8, np.zeros((2, 0), np.int8), np.ones(2, np.float32), want_acc=True)
    assert np.all(y == 0) and np.all(acc == 0)


def test_decode_every_byte_value_including_code_11():
    """A blob written by hand from the documented layout holds all 256 byte
    values (code 11 included); the product must treat 11 as 0."""
    from ternary_weight_amd import tq
    t = torch()
    N, Kin = 64, 1024
    d = tq.desc(1, 0, tq.SCALE_TENSOR, N, Kin)
    size = tq.packed_size(d)
    raw = np.zeros(size, dtype=np.uint8)
    codes = RNG.integers(0, 256, size=N * Kin // 4, dtype=np.uint8)
    codes[:256] = np.arange(256, dtype=np.uint8)
    raw[256:256 + codes.size] = codes
    s_w = np.float32(0.0625)
    end = (256 + codes.size + 255) & ~255
    raw[end:end + 4] = np.array([s_w], np.float32).view(np.uint8)
    raw[:4] = np.array([0x31575154], np.uint32).view(np.uint8)
    trits = read_blob(raw, 1, N, Kin, TENSOR)["trits"]        # 11 -> 0 by the layout's rule
    assert np.any(read_blob(raw, 1, N, Kin, TENSOR)["codes"] == 3)
    blob = dev(raw)
    x = rand_x(3, Kin, F32)
    q, s = oracle.act_quant_i8(x)
    y, acc = gemv(d, blob, I8, q, s, want_acc=True)
    ref = oracle.gemv_i8(1, 0, TENSOR, trits, np.array([s_w]), q, s)
    assert np.array_equal(acc, ref["acc"].astype(np.int32))
    assert np.array_equal(y.view(np.uint32), ref["y32"].view(np.uint32))
    xb = rand_x(2, Kin, BF16)
    yb = gemv(d, blob, BF16, xb)
    assert rel_err(yb, oracle.gemv_fp(1, 0, TENSOR, trits, np.array([s_w]), xb, BF16)) <= TOL
    xf = rand_x(2, Kin, F32)
    yf = gemv(d, blob, F32, xf)
    assert rel_err(yf, oracle.gemv_fp(1, 0, TENSOR, trits, np.array([s_w]), xf, F32)) <= TOL


def test_one_hot_activation_reads_one_column():
    K, g, N, Kin = 3, 256, 128, 1024
    trits, scales, _ = rand_problem(K, g, GROUP_F16, N, Kin)
    d, blob = pack(K, g, GROUP_F16, trits, scales)
    for j in (0, 1, 5, 63, 64, 255, 256, 1023):
        x = np.zeros((1, Kin), np.float32)
        x[0, j] = 1.0
        y = gemv(d, blob, F32, x)
        ref = oracle.gemv_fp(K, g, GROUP_F16, trits, scales, x, F32)
        assert np.allclose(y[0], ref[0], rtol=2e-7, atol=0), j


def test_deterministic_repeat():
    trits, scales, _ = rand_problem(3, 256, GROUP_F16, 4096, 4096)
    d, blob = pack(3, 256, GROUP_F16, trits, scales)
    x = rand_x(1, 4096, BF16)
    y1 = gemv(d, blob, BF16, x)
    y2 = gemv(d, blob, BF16, x)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


# ---------------------------------------------------------------------------
# Grouped launch.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("x_type,K,g,layout,M", [(I8, 1, 0, TENSOR, 1), (BF16, 3, 256, GROUP_F16, 1),
                                                  (BF16, 3, 16, CODEBOOK, 4), (F32, 2, 64, GROUP_F16, 2),
                                                  (F32_Q8, 1, 0, TENSOR, 1), (F32_Q8, 1, 0, TENSOR, 4)])
@pytest.mark.parametrize("waves,row_blocks", [(0, 0), (1, 1), (4, 1), (16, 1), (1, 4), (2, 2), (2, 8), (1, 16)])
def test_grouped_matches_oracle(x_type, K, g, layout, M, waves, row_blocks):
    from ternary_weight_amd import tq
    t = torch()
    shapes = [(640, 2560), (64, 256), (2560, 512), (130, 768), (96, 6912)]
    keep, items, refs, ys = [], [], [], []
    for i, (N, Kin) in enumerate(shapes):
        trits, scales, cb = rand_problem(K, g, layout, N, Kin)
        d, blob = pack(K, g, layout, trits, scales, cb)
        if x_type in (I8, F32_Q8):
            xf = rand_x(M, Kin, F32)
            q, s = oracle.act_quant_i8(xf)
            xd, sd = (dev(q), dev(s)) if x_type == I8 else (dev(xf), None)
            r = oracle.gemv_i8(K, g, layout, trits, scales, q, s, cb)
            refs.append(r["y32"] if layout == TENSOR and K == 1 else r["y64"])
        else:
            x = rand_x(M, Kin, x_type)
            xd, sd = dev(x), None
            refs.append(oracle.gemv_fp(K, g, layout, trits, scales, x, x_type, cb))
        y = t.full((M, N), float("nan"), dtype=t.float32, device="cuda")
        keep += [d, blob, xd, sd]
        ys.append(y)
        items.append((d, blob, xd, sd, y, None))
    probs = tq.problems(items)
    nbytes = tq.gemv_grouped_workspace_size(probs, M)
    ws = t.empty(nbytes, dtype=t.uint8, device="cuda")
    plan = tq.gemv_grouped_prepare(probs, M, x_type, ws, nbytes, waves=waves, row_blocks=row_blocks)
    if plan.family >= 1000:
        # a matrix-core plan (bf16 or int8 with several tokens): one item per 16-token x 256-row tile
        assert x_type in (BF16, I8) and M > 1
        assert plan.n_items == sum((N + 255) // 256 for N, _ in shapes)
    else:
        R = plan.row_blocks
        assert plan.n_items == sum(((N + 63) // 64 + R - 1) // R for N, _ in shapes)
        if waves:
            assert (plan.waves, plan.row_blocks) == (waves, row_blocks)
    tq.gemv_grouped_run(plan)
    t.cuda.synchronize()
    for y, r in zip(ys, refs):
        if x_type in (I8, F32_Q8) and layout == TENSOR and K == 1:
            assert np.array_equal(host(y).view(np.uint32), r.view(np.uint32))
        else:
            assert rel_err(host(y), r) <= TOL


@pytest.mark.parametrize("M", [5, 9, 16])
@pytest.mark.parametrize("x_type,shape", [(F32, (0, 0)), (F32, (2, 2)), (I8, (0, 0)), (I8, (4, 1)),
                                          (F32_Q8, (0, 0)), (F32_Q8, (2, 4)), (BF16, (1, 16)), (BF16, (0, 0))])
def test_grouped_token_slices(x_type, shape, M):
    """More tokens than a pass takes (4): each problem is cut
    into slices, with holes in the item list: bf16 without a shape hint an
    item per wave, a row block's slices in one workgroup; otherwise slices
    placed 8 workgroups apart.  bf16 (M >= 3) and int8 (M >= 2, groups of 64)
    without a shape hint go to the matrix cores; with one they stay on the
    vector ALUs."""
    from ternary_weight_amd import tq
    t = torch()
    K, g, layout = 2, 64, GROUP_F16
    shapes = [(640, 512), (64, 256), (130, 768), (200, 1024), (96, 64)]
    keep, items, refs, ys = [], [], [], []
    for i, (N, Kin) in enumerate(shapes):
        trits, scales, cb = rand_problem(K, g, layout, N, Kin)
        d, blob = pack(K, g, layout, trits, scales, cb)
        if x_type in (I8, F32_Q8):
            xf = rand_x(M, Kin, F32)
            q, s = oracle.act_quant_i8(xf)
            xd, sd = (dev(q), dev(s)) if x_type == I8 else (dev(xf), None)
            refs.append(oracle.gemv_i8(K, g, layout, trits, scales, q, s, cb)["y64"])
        else:
            x = rand_x(M, Kin, x_type)
            xd, sd = dev(x), None
            refs.append(oracle.gemv_fp(K, g, layout, trits, scales, x, x_type, cb))
        y = t.full((M, N), float("nan"), dtype=t.float32, device="cuda")
        keep += [d, blob, xd, sd]
        ys.append(y)
        items.append((d, blob, xd, sd, y, None))
    probs = tq.problems(items)
    nbytes = tq.gemv_grouped_workspace_size(probs, M)
    ws = t.empty(nbytes, dtype=t.uint8, device="cuda")
    waves, row_blocks = shape
    if x_type == BF16 and shape != (0, 0):
        plan = tq.gemv_grouped_prepare_tokens(probs, [M] * len(shapes), x_type, ws, nbytes, waves=waves,
                                              row_blocks=row_blocks)
        assert plan.family < 1000 and plan.mode == 0
    else:
        plan = tq.gemv_grouped_prepare(probs, M, x_type, ws, nbytes, waves=waves, row_blocks=row_blocks)
    if plan.family >= 1000:
        assert x_type in (BF16, I8) and shape == (0, 0)
    else:
        slices = (M + 3) // 4
        assert plan.n_problems == len(shapes) * slices
        R = plan.row_blocks
        if plan.mode == 1:
            # an item per wave, a row block's slices in one workgroup of R waves
            assert shape == (0, 0) and x_type == BF16 and R == 16
            busy = sum((N + 63) // 64 for N, _ in shapes) * slices
            assert busy <= plan.n_items <= 2 * busy + R and plan.n_items % R == 0
        else:
            busy = sum(((N + 63) // 64 + R - 1) // R for N, _ in shapes) * slices
            assert busy <= plan.n_items <= busy + 8 * (slices + 1)
    tq.gemv_grouped_run(plan)
    t.cuda.synchronize()
    for y, r in zip(ys, refs):
        assert rel_err(host(y), r) <= TOL


@pytest.mark.parametrize("N,Kin,M", [(2560, 2560, 1), (640, 2560, 1), (2560, 6912, 1), (130, 80, 3),
                                     (64, 4096, 16), (200, 65536, 1), (64, 16, 1)])
def test_fused_quantisation_is_bit_identical(N, Kin, M):
    """fp32 x quantised inside the product == tq_act_quant_int8 then the int8 product."""
    trits, scales, _ = rand_problem(1, 0, TENSOR, N, Kin)
    x = (rand_x(M, Kin, F32) * 10.0 ** float(RNG.integers(-3, 4))).astype(np.float32)
    if M > 2:
        x[1] = 0.0
    q, s = oracle.act_quant_i8(x)
    d, blob = pack(1, 0, TENSOR, trits, scales)
    y, acc = gemv(d, blob, F32_Q8, x, want_acc=True)
    ref = oracle.gemv_i8(1, 0, TENSOR, trits, scales, q, s)
    assert np.array_equal(acc, ref["acc"].astype(np.int32))
    assert np.array_equal(y.view(np.uint32), ref["y32"].view(np.uint32))


def test_act_quant_batch_bit_exact():
    from ternary_weight_amd import tq
    t = torch()
    segs, want, keep = [], [], []
    for (M, Kin, xt) in [(180, 2560, F32), (30, 6912, F32), (3, 16, BF16), (0, 64, F32), (5, 40000, F32),
                         (2, 4096, BF16)]:
        v = RNG.standard_normal((M, Kin)) * 10.0 ** RNG.uniform(-5, 5, size=(M, 1))
        if M > 1:
            v[0] = 0.0
        x = gen.bf16_bits(v) if xt == BF16 else v.astype(np.float32)
        xd = dev(x)
        qd = t.full((M, Kin), 99, dtype=t.int8, device="cuda")
        sd = t.full((M,), -1.0, dtype=t.float32, device="cuda")
        keep.append((xd, qd, sd))
        segs.append((M, Kin, xt, xd, qd, sd))
        want.append(oracle.act_quant_i8(x, xt) if M else None)
    tq.act_quant_int8_batch(segs)
    t.cuda.synchronize()
    for (xd, qd, sd), w in zip(keep, want):
        if w is None:
            continue
        assert np.array_equal(host(qd), w[0])
        assert np.array_equal(host(sd).view(np.uint32), w[1].view(np.uint32))
