"""GPU parity of the prefill product (tq_gemm, tq_gemm_grouped_*) against the
CPU oracle, through the C ABI.

Bars as for decode: bit-exact y and int32 accumulator for int8 activations
with one plane and a per-tensor scale; the per-token relative error
max_n |y - y*| / max(|y*|, rms(y*)) <= 1e-3 against the fp64 oracle otherwise.
Sizes span several 128 x 128 output tiles (16 x 256 for bf16 with M <= 16)
with ragged edges in M, N and Kin.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle import BF16, CODEBOOK, F32, GROUP_F16, I8, TENSOR
from synth import gen
from tests.gpu_util import TOL, dev, gemv, host, pack, read_blob, rel_err, torch
from tests.test_gpu_parity import rand_problem, rand_x

pytestmark = pytest.mark.gpu


def check_i8(K, g, layout, trits, scales, d, blob, q, s, exact):
    ref = oracle.gemv_i8(K, g, layout, trits, scales, q, s)
    if exact:
        y, acc = gemv(d, blob, I8, q, s, want_acc=True, gemm=True)
        assert np.array_equal(acc.astype(np.int64), ref["acc"].reshape(acc.shape))
        assert np.array_equal(y.view(np.uint32), ref["y32"].view(np.uint32))
    else:
        y = gemv(d, blob, I8, q, s, gemm=True)
        assert rel_err(y, ref["y64"]) <= TOL


@pytest.mark.parametrize("N,Kin,M", [
    (256, 512, 128), (200, 80, 17), (640, 2560, 300), (64, 64, 1), (513, 1024, 129), (1, 16, 5),
])
def test_gemm_i8_tensor_bit_exact(N, Kin, M):
    rng = np.random.default_rng(N * 7 + Kin + M)
    trits, scales, _ = rand_problem(1, 0, TENSOR, N, Kin, rng)
    d, blob = pack(1, 0, TENSOR, trits, scales)
    q, s = oracle.act_quant_i8(rand_x(M, Kin, F32, rng))
    check_i8(1, 0, TENSOR, trits, scales, d, blob, q, s, exact=True)


def test_gemm_i8_extreme_accumulators():
    # every trit +1 against x at +-127: |acc| = 127 * Kin, the largest the format allows here
    N, Kin, M = 130, 4096, 70
    trits = np.ones((1, N, Kin), dtype=np.int8)
    trits[0, 1::2] = -1
    scales = np.array([0.0123], dtype=np.float32)
    d, blob = pack(1, 0, TENSOR, trits, scales)
    x = np.full((M, Kin), 3.5, dtype=np.float32)
    x[1::2] = -3.5
    q, s = oracle.act_quant_i8(x)
    assert np.abs(q).max() == 127
    check_i8(1, 0, TENSOR, trits, scales, d, blob, q, s, exact=True)


@pytest.mark.parametrize("K,g,layout", [
    (2, 0, TENSOR), (3, 0, TENSOR), (4, 0, TENSOR),
    (1, 64, GROUP_F16), (3, 128, GROUP_F16), (2, 256, GROUP_F16), (4, 64, GROUP_F16),
])
def test_gemm_i8_other_layouts(K, g, layout):
    rng = np.random.default_rng(K * 100 + g + layout)
    N, Kin, M = 200, 768, 140
    trits, scales, _ = rand_problem(K, g, layout, N, Kin, rng)
    d, blob = pack(K, g, layout, trits, scales)
    q, s = oracle.act_quant_i8(rand_x(M, Kin, F32, rng))
    check_i8(K, g, layout, trits, scales, d, blob, q, s, exact=False)


@pytest.mark.parametrize("K,g,layout", [
    (1, 0, TENSOR), (3, 0, TENSOR), (1, 32, GROUP_F16), (3, 256, GROUP_F16), (2, 64, GROUP_F16),
    (4, 128, GROUP_F16), (3, 32, GROUP_F16), (2, 16, GROUP_F16), (3, 16, CODEBOOK), (3, 32, CODEBOOK),
    (2, 64, CODEBOOK), (1, 16, CODEBOOK),
])
@pytest.mark.parametrize("N,Kin,M", [(200, 768, 140), (64, 256, 1), (300, 1280, 37), (130, 512, 16), (70, 512, 5)])
def test_gemm_bf16(K, g, layout, N, Kin, M):
    # M <= 16 runs the one-tile (1 x 4 waves) kernels, larger M the 2 x 2 ones
    rng = np.random.default_rng(K * 1000 + g + N + M)
    trits, scales, cb = rand_problem(K, g, layout, N, Kin, rng)
    d, blob = pack(K, g, layout, trits, scales, cb)
    x = rand_x(M, Kin, BF16, rng)
    y = gemv(d, blob, BF16, x, gemm=True)
    ref = oracle.gemv_fp(K, g, layout, trits, scales, x, BF16, cb)
    err = rel_err(y, ref)
    assert err <= TOL, err
    assert err <= 1e-5          # fp32 accumulation is far inside the bar


def test_gemm_ragged_kin_tail():
    # Kin not a multiple of the MFMA step: the last step is part padding
    rng = np.random.default_rng(5)
    for (Kin, xt) in ((80, I8), (48, BF16), (16, I8), (16, BF16), (1040, I8)):
        N, M = 70, 33
        trits, scales, _ = rand_problem(1, 0, TENSOR, N, Kin, rng)
        d, blob = pack(1, 0, TENSOR, trits, scales)
        if xt == I8:
            q, s = oracle.act_quant_i8(rand_x(M, Kin, F32, rng))
            check_i8(1, 0, TENSOR, trits, scales, d, blob, q, s, exact=True)
        else:
            x = rand_x(M, Kin, BF16, rng)
            assert rel_err(gemv(d, blob, BF16, x, gemm=True), oracle.gemv_fp(1, 0, TENSOR, trits, scales, x, BF16)) <= TOL


@pytest.mark.parametrize("M", [3, 16, 40])
@pytest.mark.parametrize("Kin,K", [(48, 1), (80, 3), (1008, 2)])
def test_ragged_kin_ignores_the_next_tokens_infinity(M, Kin, K):
    """bf16 x, per-tensor scale, Kin not a multiple of the 32-column MFMA
    step: the last step's columns past Kin lie in the next token's row.  An
    infinity at the start of token 1 must leave every other token finite and
    equal to the oracle (which takes finite inputs only: its reference has
    token 1 zeroed, which no other token depends on).  M = 3 and 16 run the
    few-token kernels (tq_gemv and tq_gemm), M = 40 the prefill kernels."""
    rng = np.random.default_rng(Kin + M + K)
    N = 70
    trits, scales, _ = rand_problem(K, 0, TENSOR, N, Kin, rng)
    d, blob = pack(K, 0, TENSOR, trits, scales)
    v = rng.standard_normal((M, Kin))
    v[1] = 0.0
    ref = oracle.gemv_fp(K, 0, TENSOR, trits, scales, gen.bf16_bits(v), BF16)
    v[1, :3] = [np.inf, -np.inf, np.inf]
    x = gen.bf16_bits(v)
    keep = [m for m in range(M) if m != 1]
    for y in (gemv(d, blob, BF16, x, gemm=True), gemv(d, blob, BF16, x) if M <= 16 else None):
        if y is None:
            continue
        assert np.all(np.isfinite(y[keep]))
        assert rel_err(y[keep], ref[keep]) <= TOL


def test_gemm_one_hot_indexing():
    # x = e_j picks column j: y[j][n] = s[n][j / g] * t[n][j] exactly, for every
    # j of a row of two groups and every n of two weight tiles
    N, Kin = 96, 128
    rng = np.random.default_rng(9)
    trits, scales, _ = rand_problem(1, 64, GROUP_F16, N, Kin, rng)
    d, blob = pack(1, 64, GROUP_F16, trits, scales)
    x = np.zeros((Kin, Kin), dtype=np.float32)
    np.fill_diagonal(x, 1.0)
    from synth import gen
    y = gemv(d, blob, BF16, gen.bf16_bits(x), gemm=True)
    s = np.array([[oracle.f16_to_f64(int(h)) for h in row] for row in scales[0]])   # [N][G]
    want = (s[:, np.arange(Kin) // 64] * trits[0]).T                                   # [Kin][N]
    assert np.array_equal(y, want.astype(np.float32))


def test_gemm_matches_gemv_at_small_m():
    # the two kernel families agree where both apply (int8: bit for bit)
    rng = np.random.default_rng(11)
    N, Kin, M = 320, 2560, 3
    trits, scales, _ = rand_problem(1, 0, TENSOR, N, Kin, rng)
    d, blob = pack(1, 0, TENSOR, trits, scales)
    q, s = oracle.act_quant_i8(rand_x(M, Kin, F32, rng))
    a = gemv(d, blob, I8, q, s, want_acc=True)
    b = gemv(d, blob, I8, q, s, want_acc=True, gemm=True)
    assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32)) and np.array_equal(a[1], b[1])


def test_gemm_unsupported_and_empty():
    from ternary_weight_amd import tq
    t = torch()
    trits, scales, cb = rand_problem(3, 16, CODEBOOK, 64, 64)
    d, blob = pack(3, 16, CODEBOOK, trits, scales, cb)
    xq = t.zeros((4, 64), dtype=t.int8, device="cuda")
    xs = t.ones(4, dtype=t.float32, device="cuda")
    y = t.zeros((4, 64), dtype=t.float32, device="cuda")
    with pytest.raises(tq.TQError) as e:
        tq.gemm(d, blob, 4, I8, xq, xs, y)           # the codec's groups of 16 are below the int8 step
    assert e.value.status == tq.ERR_UNSUPPORTED
    trits, scales, _ = rand_problem(1, 32, GROUP_F16, 64, 64)
    d, blob = pack(1, 32, GROUP_F16, trits, scales)
    with pytest.raises(tq.TQError) as e:
        tq.gemm(d, blob, 4, I8, xq, xs, y)          # g = 32 is below the int8 MFMA step
    assert e.value.status == tq.ERR_UNSUPPORTED
    with pytest.raises(tq.TQError) as e:
        tq.gemm(d, blob, 4, F32, t.zeros((4, 64), device="cuda"), None, y)
    assert e.value.status == tq.ERR_UNSUPPORTED
    tq.gemm(d, blob, 0, BF16, None, None, None)       # M = 0: no-op
    t.cuda.synchronize()


def test_gemm_deterministic():
    rng = np.random.default_rng(21)
    trits, scales, _ = rand_problem(3, 256, GROUP_F16, 700, 2048, rng)
    d, blob = pack(3, 256, GROUP_F16, trits, scales)
    x = rand_x(100, 2048, BF16, rng)
    a = gemv(d, blob, BF16, x, gemm=True)
    b = gemv(d, blob, BF16, x, gemm=True)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("xt,K,g,layout", [(I8, 1, 0, TENSOR), (BF16, 3, 256, GROUP_F16), (I8, 2, 64, GROUP_F16),
                                            (BF16, 3, 16, CODEBOOK)])
def test_gemm_grouped_equals_single(xt, K, g, layout):
    from ternary_weight_amd import tq
    t = torch()
    rng = np.random.default_rng(31 + K)
    M = 77
    shapes = [(256, 512), (64, 1024), (700, 256), (130, 768)]
    keep, items, want = [], [], []
    for (N, Kin) in shapes:
        trits, scales, cb = rand_problem(K, g, layout, N, Kin, rng)
        d, blob = pack(K, g, layout, trits, scales, cb)
        if xt == I8:
            q, s = oracle.act_quant_i8(rand_x(M, Kin, F32, rng))
            xd, xs = dev(q), dev(s)
        else:
            xd, xs = dev(rand_x(M, Kin, BF16, rng)), None
        y = t.full((M, N), float("nan"), dtype=t.float32, device="cuda")
        keep.append((d, blob, xd, xs, y))
        items.append((d, blob, xd, xs, y, None))
        want.append(gemv(d, blob, xt, xd, xs, gemm=True))
    probs = tq.problems(items)
    n = tq.gemm_grouped_workspace_size(probs, M, xt)
    ws = t.empty(n, dtype=t.uint8, device="cuda")
    plan = tq.gemm_grouped_prepare(probs, M, xt, ws, n)
    for _ in range(2):
        tq.gemm_grouped_run(plan)
        t.cuda.synchronize()
        for (d, blob, xd, xs, y), w in zip(keep, want):
            assert np.array_equal(host(y).view(np.uint32), w.view(np.uint32))
    # the decode run executes a matrix-core plan too (it prepares them for bf16 with several tokens)
    for (d, blob, xd, xs, y) in keep:
        y.fill_(float("nan"))
    tq.gemv_grouped_run(plan)
    t.cuda.synchronize()
    for (d, blob, xd, xs, y), w in zip(keep, want):
        assert np.array_equal(host(y).view(np.uint32), w.view(np.uint32))


@pytest.mark.parametrize("layout,K,g", [(CODEBOOK, 3, 16), (GROUP_F16, 3, 256), (GROUP_F16, 2, 16)])
@pytest.mark.parametrize("M", [2, 3, 4, 5, 9, 16])
def test_decode_bf16_several_tokens_on_matrix_cores(layout, K, g, M):
    """tq_gemv and the grouped decode plan route bf16 with 3 or more tokens
    (the codec's digit planes included) to the one-tile matrix-core kernels,
    fewer to the vector ALUs in slices of 4; both agree with the oracle, and on
    the matrix cores the grouped plan bit for bit with the single call."""
    from ternary_weight_amd import tq
    t = torch()
    rng = np.random.default_rng(M * 10 + g + K)
    shapes = [(1024, 512), (320, 1024), (96, 256)]
    keep, items, want = [], [], []
    for (N, Kin) in shapes:
        trits, scales, cb = rand_problem(K, g, layout, N, Kin, rng)
        d, blob = pack(K, g, layout, trits, scales, cb)
        x = rand_x(M, Kin, BF16, rng)
        y1 = gemv(d, blob, BF16, x)
        assert rel_err(y1, oracle.gemv_fp(K, g, layout, trits, scales, x, BF16, cb)) <= TOL
        xd = dev(x)
        y = t.full((M, N), float("nan"), dtype=t.float32, device="cuda")
        keep.append((d, blob, xd, y))
        items.append((d, blob, xd, None, y, None))
        want.append(y1)
    probs = tq.problems(items)
    n = tq.gemv_grouped_workspace_size(probs, M)
    ws = t.empty(n, dtype=t.uint8, device="cuda")
    plan = tq.gemv_grouped_prepare(probs, M, BF16, ws, n)
    on_mfma = M >= 3
    assert (plan.family >= 1000) == on_mfma          # a matrix-core plan, or the vector ALUs
    tq.gemv_grouped_run(plan)
    t.cuda.synchronize()
    for (d, blob, xd, y), w in zip(keep, want):
        if on_mfma:
            assert np.array_equal(host(y).view(np.uint32), w.view(np.uint32))
        else:
            assert rel_err(host(y), w) <= TOL


@pytest.mark.parametrize("M", [3, 16, 40])
def test_codec_digit_planes_code_11_and_ragged_chunk(M):
    """The codec's three two-bit digit planes on the matrix cores, combined
    per column into one operand (d3 card, "Quantization details": value
    9 t2 + 3 t1 + t0), in the few-token kernel (3 and 16 tokens) and the
    prefill kernel (40): digit code 11 planted at random in every plane reads
    as 0 (the layout's rule, applied by the independent blob reader), and rows
    of 464 columns end 16 columns into their eighth 64-column chunk."""
    rng = np.random.default_rng(71 + M)
    K, g, N, Kin = 3, 16, 200, 464
    trits, scales, cb = rand_problem(K, g, CODEBOOK, N, Kin, rng)
    d, blob = pack(K, g, CODEBOOK, trits, scales, cb)
    raw = host(blob).view(np.uint8).copy()
    NB, NC = (N + 63) // 64, (Kin + 63) // 64
    nbytes = NB * NC * K * 64 * 16
    region = raw[256:256 + nbytes]
    hit = rng.random(nbytes) < 0.25
    field = rng.integers(0, 4, size=nbytes).astype(np.uint8)
    region[hit] |= (np.uint8(3) << (2 * field[hit])).astype(np.uint8)
    raw[256:256 + nbytes] = region
    rb = read_blob(raw, K, N, Kin, CODEBOOK, g=g)
    assert np.any(rb["codes"][:, :N, :Kin] == 3)
    assert np.array_equal(rb["scales"], scales)
    x = rand_x(M, Kin, BF16, rng)
    y = gemv(d, dev(raw), BF16, x, gemm=M > 16)
    assert rel_err(y, oracle.gemv_fp(K, g, CODEBOOK, rb["trits"], scales, x, BF16, cb)) <= TOL


@pytest.mark.parametrize("x_type,K,g,layout", [
    (I8, 1, 0, TENSOR), (I8, 3, 256, GROUP_F16), (BF16, 3, 256, GROUP_F16), (BF16, 3, 16, CODEBOOK),
    (BF16, 1, 16, CODEBOOK),
])
@pytest.mark.parametrize("M,N", [(17, 200), (129, 513), (300, 640), (40, 1)])
def test_gemm_writes_nothing_past_y(x_type, K, g, layout, M, N):
    """The prefill kernels store y (and the int32 sums) through a buffer
    resource the size of y and drop every output past M or N: a guard region
    after y (and after acc) keeps its sentinel, and y is right, for ragged
    token and row counts in every kernel family."""
    from ternary_weight_amd import tq
    t = torch()
    Kin = 512
    rng = np.random.default_rng(M * 31 + N + K)
    trits, scales, cb = rand_problem(K, g, layout, N, Kin, rng)
    d, blob = pack(K, g, layout, trits, scales, cb)
    guard = 8192
    ybuf = t.full((M * N + guard,), float("nan"), dtype=t.float32, device="cuda")
    abuf = t.full((M * N + guard,), -777, dtype=t.int32, device="cuda")
    want_acc = x_type == I8 and K == 1 and layout == TENSOR
    if x_type == I8:
        q, s = oracle.act_quant_i8(rand_x(M, Kin, F32, rng))
        tq.gemm(d, blob, M, I8, dev(q), dev(s), ybuf, abuf if want_acc else None)
        ref = oracle.gemv_i8(K, g, layout, trits, scales, q, s)
        want = ref["y32"] if want_acc else ref["y64"]
    else:
        x = rand_x(M, Kin, BF16, rng)
        tq.gemm(d, blob, M, BF16, dev(x), None, ybuf, None)
        want = oracle.gemv_fp(K, g, layout, trits, scales, x, BF16, cb)
    t.cuda.synchronize()
    yh = host(ybuf)
    assert np.all(np.isnan(yh[M * N:])), "a store past y"
    y = yh[:M * N].reshape(M, N)
    if want_acc:
        assert np.array_equal(y.view(np.uint32), want.view(np.uint32))
        ah = host(abuf)
        assert np.all(ah[M * N:] == -777), "a store past acc"
        assert np.array_equal(ah[:M * N].reshape(M, N), ref["acc"].astype(np.int32))
    else:
        assert rel_err(y, want) <= TOL


def test_bf16_several_tokens_weight_over_4gib_runs_on_vector_alus():
    """A bf16 call with several tokens whose codes exceed the 4 GiB that the
    matrix-core kernels address goes to the vector-ALU kernels (tq_gemv and
    the grouped plan) instead of failing: K = 3, g = 256, 1,400,017 x 4096
    (4.3 GB of codes), 3 tokens, 64 sampled rows against the oracle."""
    import torch
    from synth import device
    from ternary_weight_amd import tq
    K, g, N, Kin, M = 3, 256, 1_400_017, 4096, 3
    print("bf16 K=3 %d x %d M=%d (codes over 4 GiB)" % (N, Kin, M), flush=True)
    seed = 0x5EED4
    trits = torch.empty((K, N, Kin), dtype=torch.int8, device="cuda")
    device.fill(device.K_TRITS, seed, 0, trits)
    lo, span = gen.log_uniform_params(1e-3, 1e-1)
    sc = torch.empty((K, N, Kin // g), dtype=torch.int16, device="cuda")
    device.fill(device.K_LOGU_F16, seed + 1, 0, sc, a=lo, b=span)
    x = torch.empty((M, Kin), dtype=torch.int16, device="cuda")
    device.fill(device.K_NORMAL_BF16, seed + 2, 0, x)
    d = tq.desc(K, g, GROUP_F16, N, Kin)
    blob = torch.empty(tq.packed_size(d), dtype=torch.uint8, device="cuda")
    assert tq.packed_size(d) > (1 << 32)
    tq.pack(d, trits, sc, None, blob)
    rows = np.sort(np.random.default_rng(3).choice(N, size=64, replace=False))
    rows[-1] = N - 1
    ridx = torch.from_numpy(rows).cuda()
    t_h = trits.index_select(1, ridx).cpu().numpy()
    s_h = sc.index_select(1, ridx).cpu().numpy().view(np.uint16)
    x_h = x.cpu().numpy().view(np.uint16)
    del trits
    torch.cuda.empty_cache()
    ref = oracle.gemv_fp(K, g, GROUP_F16, t_h, s_h, x_h, BF16)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    tq.gemv(d, blob, M, BF16, x, None, y)
    torch.cuda.synchronize()
    assert rel_err(y[:, ridx].cpu().numpy(), ref) <= TOL
    y2 = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    probs = tq.problems([(d, blob, x, None, y2, None)])
    ws = torch.empty(tq.gemv_grouped_workspace_size(probs, M), dtype=torch.uint8, device="cuda")
    plan = tq.gemv_grouped_prepare(probs, M, BF16, ws, ws.numel())
    assert plan.family < 1000            # a vector-ALU plan
    tq.gemv_grouped_run(plan)
    torch.cuda.synchronize()
    assert rel_err(y2[:, ridx].cpu().numpy(), ref) <= TOL
    del blob, y, y2, ws
    torch.cuda.empty_cache()
