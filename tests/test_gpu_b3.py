"""The codec with compact base-3 codes (TQ_SCALE_CODEBOOK_B3) on the GPU:
packing against the independent reader of the documented layout, every one
of the 729 pair codes, the round trip through tq_unpack, and the products
(vector-ALU decode, matrix-core decode and prefill, grouped plans) against
the CPU oracle of the codec -- the same definition and canonical arrays as
TQ_SCALE_CODEBOOK, whose results these equal within the bound."""
from __future__ import annotations

import itertools

import numpy as np
import pytest

import oracle
from oracle import BF16, CODEBOOK
from synth import gen
from tests.gpu_util import TOL, dev, gemv, host, read_blob, rel_err, torch

pytestmark = pytest.mark.gpu
B3 = 3
CB = gen.codebook_f16(27)


def _digits(rng, N, Kin):
    return rng.integers(-1, 2, size=(3, N, Kin)).astype(np.int8)


def _pack(trits, idx, layout=B3):
    from ternary_weight_amd import tq
    _, N, Kin = trits.shape
    g = Kin // idx.shape[1]
    d = tq.desc(3, g, layout, N, Kin, n_codebook=27)
    blob = torch().empty(tq.packed_size(d), dtype=torch().uint8, device="cuda")
    tq.pack(d, dev(trits), dev(idx), dev(CB), blob)
    return d, blob


@pytest.mark.parametrize("N,Kin,g", [(64, 64, 16), (130, 208, 16), (7, 96, 32), (200, 1024, 64), (65, 512, 256)])
def test_pack_layout_and_roundtrip(N, Kin, g):
    from ternary_weight_amd import tq
    rng = np.random.default_rng(N * 7 + Kin)
    trits = _digits(rng, N, Kin)
    idx = rng.integers(0, 27, size=(N, Kin // g)).astype(np.uint8)
    d, blob = _pack(trits, idx)
    got = read_blob(host(blob), 3, N, Kin, B3, g)
    assert np.array_equal(got["trits"], trits)
    assert np.array_equal(got["scales"], idx)
    assert np.array_equal(got["codebook"][:27], CB)
    assert got["codes"].max() < 729                     # codes 729.. are never written
    t = torch()
    back = t.full((3, N, Kin), 5, dtype=t.int8, device="cuda")
    sc = t.zeros((N, Kin // g), dtype=t.uint8, device="cuda")
    cb = t.zeros(27, dtype=t.int16, device="cuda")
    tq.unpack(d, blob, back, sc, cb)
    t.cuda.synchronize()
    assert np.array_equal(host(back), trits)
    assert np.array_equal(host(sc), idx)
    assert np.array_equal(host(cb).view(np.uint16), CB)


def test_all_729_pair_codes():
    """Row n, pair j holds the values (a, b) of code j: every code once, checked
    through the reader and the product (one-hot activations read columns)."""
    vals = {}
    for t0, t1, t2 in itertools.product((-1, 0, 1), repeat=3):
        vals[9 * t0 + 3 * t1 + t2] = (t0, t1, t2)
    Kin = 1472                                            # 736 pairs, a multiple of 16 columns
    trits = np.zeros((3, 64, Kin), dtype=np.int8)
    want_codes = np.zeros(Kin // 2, dtype=np.int64)
    for j, (a, b) in enumerate(itertools.product(range(-13, 14), repeat=2)):
        trits[:, 0, 2 * j] = vals[a]
        trits[:, 0, 2 * j + 1] = vals[b]
        want_codes[j] = (a % 27) + 27 * (b % 27)
    trits[:, 1:] = trits[:, :1]
    idx = np.full((64, Kin // 16), 26, dtype=np.uint8)
    d, blob = _pack(trits, idx)
    got = read_blob(host(blob), 3, 64, Kin, B3, 16)
    assert np.array_equal(got["codes"][0, :Kin // 2], want_codes)
    assert sorted(got["codes"][0, :729]) == list(range(729))
    # the product with x = 1 in every column equals the oracle's (sum of every value times the scale)
    x = gen.bf16_bits(np.ones((1, Kin)))
    y = gemv(d, blob, BF16, x)
    ref = oracle.gemv_fp(3, 16, CODEBOOK, trits, idx, x, BF16, CB)
    assert rel_err(y, ref) <= TOL


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 13, 16])
@pytest.mark.parametrize("N,Kin,g", [(256, 512, 16), (130, 208, 16), (300, 1024, 64), (64, 256, 256)])
def test_gemv_matches_oracle(M, N, Kin, g):
    rng = np.random.default_rng(M * 1000 + N)
    trits = _digits(rng, N, Kin)
    idx = rng.integers(0, 27, size=(N, Kin // g)).astype(np.uint8)
    x = gen.bf16_bits(rng.standard_normal((M, Kin)))
    d, blob = _pack(trits, idx)
    y = gemv(d, blob, BF16, x)
    ref = oracle.gemv_fp(3, g, CODEBOOK, trits, idx, x, BF16, CB)
    assert rel_err(y, ref) <= TOL
    # the same weight in the two-bit-plane codec layout gives the same product within the bound
    d2, blob2 = _pack(trits, idx, CODEBOOK)
    assert rel_err(gemv(d2, blob2, BF16, x), ref) <= TOL


@pytest.mark.parametrize("M", [17, 100, 512])
@pytest.mark.parametrize("N,Kin,g", [(256, 512, 16), (200, 208, 16), (300, 1024, 32)])
def test_gemm_matches_oracle(M, N, Kin, g):
    rng = np.random.default_rng(M + N + g)
    trits = _digits(rng, N, Kin)
    idx = rng.integers(0, 27, size=(N, Kin // g)).astype(np.uint8)
    x = gen.bf16_bits(rng.standard_normal((M, Kin)))
    d, blob = _pack(trits, idx)
    y = gemv(d, blob, BF16, x, gemm=True)
    assert rel_err(y, oracle.gemv_fp(3, g, CODEBOOK, trits, idx, x, BF16, CB)) <= TOL


def test_one_hot_columns():
    """x = e_j reads column j of every row exactly: cb[idx] (9 t0 + 3 t1 + t2)."""
    rng = np.random.default_rng(9)
    N, Kin = 96, 320
    trits = _digits(rng, N, Kin)
    idx = rng.integers(0, 27, size=(N, Kin // 16)).astype(np.uint8)
    d, blob = _pack(trits, idx)
    cbf = np.array([oracle.f16_to_f64(int(h)) for h in CB])
    for j in (0, 1, 15, 16, 63, 64, 65, 127, 200, 319):
        x = np.zeros((1, Kin))
        x[0, j] = 1.0
        want = cbf[idx[:, j // 16]] * (9.0 * trits[0, :, j] + 3.0 * trits[1, :, j] + trits[2, :, j])
        for gm in (False, True):
            y = gemv(d, blob, BF16, gen.bf16_bits(x), gemm=gm) if not gm else \
                gemv(d, blob, BF16, gen.bf16_bits(np.repeat(x, 20, axis=0)), gemm=True)[:1]
            assert np.array_equal(y[0].astype(np.float64), want.astype(np.float32).astype(np.float64)), (j, gm)


@pytest.mark.parametrize("M", [1, 4, 8, 16])
def test_grouped_plan_matches_oracle(M):
    from ternary_weight_amd import tq
    t = torch()
    rng = np.random.default_rng(40 + M)
    shapes = [(256, 512), (130, 1024), (64, 208)]
    items, refs, keep = [], [], []
    for (N, Kin) in shapes:
        trits = _digits(rng, N, Kin)
        idx = rng.integers(0, 27, size=(N, Kin // 16)).astype(np.uint8)
        x = gen.bf16_bits(rng.standard_normal((M, Kin)))
        d, blob = _pack(trits, idx)
        xd = dev(x)
        y = t.full((M, N), float("nan"), dtype=t.float32, device="cuda")
        keep += [d, blob, xd, y]
        items.append((d, blob, xd, None, y, None))
        refs.append(oracle.gemv_fp(3, 16, CODEBOOK, trits, idx, x, BF16, CB))
    probs = tq.problems(items)
    ws = t.empty(tq.gemv_grouped_workspace_size(probs, M), dtype=t.uint8, device="cuda")
    plan = tq.gemv_grouped_prepare(probs, M, BF16, ws, ws.numel())
    tq.gemv_grouped_run(plan)
    t.cuda.synchronize()
    for (_, _, _, _, y, _), ref in zip(items, refs):
        assert rel_err(host(y), ref) <= TOL
