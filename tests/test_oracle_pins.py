"""Pins of the CPU oracle against things other than itself (no GPU).

The oracle (oracle/oracle.c) writes out the definition
    y[m][n] = sum_k sum_g S_k[n][g] * sum_{i in g} t_k[n][i] * x[m][i].
These tests hold it to:
  * the dense "fake-quant" product: dequantise W in fp64 with numpy and call
    numpy's matmul (sasori page, "g (group-size)": the kernel reproduces the
    fake-quant result; model card, "Quick load": FP16-dequantised weights);
  * the balanced-ternary codec written the card's way, one integer digit value
    9 t2 + 3 t1 + t0 per weight times the codebook scale;
  * closed forms and invariants (one-hot inputs, identity planes, all-ones,
    zeros, permutations, power-of-two scaling, sign);
  * library routines (numpy float16 decoding of all 65536 patterns);
  * the quantiser's defining properties (error bound, argmax at 127, symmetry,
    ties to even, scale invariance);
and a mutation check plants typical mistakes in a copy of oracle.c and
requires each to fail at least one pin.
"""
from __future__ import annotations

import json
import math
import os
import re
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from oracle import BF16, CODEBOOK, F32, GROUP_F16, TENSOR
from synth import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(20261203)


# ---------------------------------------------------------------------------
# Independent formulations used as pins.
# ---------------------------------------------------------------------------
def dense_weight(K, g, layout, trits, scales, codebook):
    """fp64 dequantised W [N][Kin] built the dense way."""
    t = trits.astype(np.float64)
    _, N, Kin = t.shape
    if layout == TENSOR:
        return np.einsum("k,kni->ni", scales.astype(np.float64), t)
    if layout == GROUP_F16:
        S = scales.view(np.float16).astype(np.float64)          # [K][N][G]
        S = np.repeat(S, g, axis=2)                              # [K][N][Kin]
        return (S * t).sum(axis=0)
    # codebook: one integer level per weight (9 t2 + 3 t1 + t0 for d = 3),
    # plane 0 the most significant digit, times the group's codebook scale.
    level = np.zeros((N, Kin), dtype=np.int64)
    for k in range(K):
        level = level * 3 + trits[k].astype(np.int64)
    cb = codebook.view(np.float16).astype(np.float64)
    S = np.repeat(cb[scales.astype(np.int64)], g, axis=1)        # [N][Kin]
    return S * level.astype(np.float64)


def x_f64(x, x_type):
    if x_type == BF16:
        return gen.bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def random_problem(K, g, layout, N, Kin, M, x_type, rng=RNG):
    trits = rng.choice(np.array([-1, 0, 1], dtype=np.int8), size=(K, N, Kin), p=[0.3, 0.4, 0.3])
    codebook = None
    if layout == TENSOR:
        scales = (10 ** rng.uniform(-3, -1, size=K)).astype(np.float32)
    elif layout == GROUP_F16:
        scales = gen.f16_bits(10 ** rng.uniform(-3, -1, size=(K, N, Kin // g)))
    else:
        scales = rng.integers(0, 27, size=(N, Kin // g), dtype=np.uint8)
        codebook = gen.codebook_f16(27)
    xv = rng.standard_normal((M, Kin))
    x = gen.bf16_bits(xv) if x_type == BF16 else xv.astype(np.float32)
    return trits, scales, codebook, x


CASES = []
for layout in (TENSOR, GROUP_F16, CODEBOOK):
    for K in (1, 2, 3, 4):
        for g in ((0,) if layout == TENSOR else (16, 32, 64, 128, 256)):
            if layout == CODEBOOK and g not in (16, 32):
                continue
            CASES.append((layout, K, g))


def check_dense(orc, layout, K, g, x_type=F32, N=24, Kin=512, M=3, rng=RNG):
    trits, scales, codebook, x = random_problem(K, g, layout, N, Kin, M, x_type, rng)
    y = orc.gemv_fp(K, g, layout, trits, scales, x, x_type, codebook)
    W = dense_weight(K, g, layout, trits, scales, codebook)
    xd = x_f64(x, x_type)
    yd = xd @ W.T
    bound = np.abs(xd) @ np.abs(W).T
    err = np.abs(y - yd)
    assert np.all(err <= 1e-13 * bound + 1e-300), (layout, K, g, float(np.max(err / (bound + 1e-300))))


def check_dense_i8(orc, layout, K, g, N=20, Kin=512, M=3, rng=RNG):
    trits, scales, codebook, _ = random_problem(K, g, layout, N, Kin, M, F32, rng)
    q = rng.integers(-127, 128, size=(M, Kin), dtype=np.int8)
    s = (10 ** rng.uniform(-4, -1, size=M)).astype(np.float32)
    out = orc.gemv_i8(K, g, layout, trits, scales, q, s, codebook)
    acc = sum(q.astype(np.int64) @ trits[k].astype(np.int64).T for k in range(K))
    assert np.array_equal(out["acc"], acc)
    W = dense_weight(K, g, layout, trits, scales, codebook)
    yd = (q.astype(np.float64) @ W.T) * s.astype(np.float64)[:, None]
    bound = (np.abs(q.astype(np.float64)) @ np.abs(W).T) * s.astype(np.float64)[:, None]
    assert np.all(np.abs(out["y64"] - yd) <= 1e-13 * bound + 1e-300)
    if layout == TENSOR and K == 1:
        exact = acc.astype(np.float64) * float(scales[0]) * s.astype(np.float64)[:, None]
        y32 = out["y32"].astype(np.float64)
        # two fp32 roundings of the real product
        assert np.all(np.abs(y32 - exact) <= 2.0 ** -23 * np.abs(exact) + 1e-45)
        # the stated order: c = fl32(s_w * s_x), then fl32(acc * c).  Each
        # product of two fp32 values (and of |acc| < 2^24 with an fp32) is exact
        # in fp64, so one rounding of the fp64 product is the fp32 result.
        c = (np.float64(scales[0]) * s.astype(np.float64)).astype(np.float32)
        want = (acc.astype(np.float64) * c.astype(np.float64)[:, None]).astype(np.float32)
        assert np.array_equal(out["y32"], want)


def check_one_hot(orc, layout, K, g, N=16, rng=RNG):
    Kin = 2 * max(g, 64)
    trits, scales, codebook, _ = random_problem(K, g, layout, N, Kin, 1, F32, rng)
    for j in (0, 1, g - 1 if g else 5, g if g else 17, Kin - 1, int(rng.integers(Kin))):
        x = np.zeros((1, Kin), dtype=np.float32)
        x[0, j] = 1.0
        y = orc.gemv_fp(K, g, layout, trits, scales, x, F32, codebook)[0]
        want = np.zeros(N)
        for k in range(K):
            if layout == TENSOR:
                S = np.full(N, float(scales[k]))
            elif layout == GROUP_F16:
                S = scales[k, :, j // g].view(np.float16).astype(np.float64)
            else:
                S = (3.0 ** (K - 1 - k)) * codebook.view(np.float16).astype(np.float64)[
                    scales[:, j // g].astype(np.int64)]
            want += S * trits[k, :, j]
        assert np.array_equal(y, want), (layout, K, g, j)


def check_quant(orc, rng=RNG):
    x = rng.standard_normal((6, 1000)).astype(np.float32) * np.float32(3.0)
    x[1] *= np.float32(1e-30)
    x[2, :] = 0.0
    q, s = orc.act_quant_i8(x)
    for m in range(x.shape[0]):
        a = float(np.max(np.abs(x[m].astype(np.float64))))
        if a == 0.0:
            assert np.all(q[m] == 0) and s[m] == 0.0
            continue
        real = x[m].astype(np.float64) * 127.0 / a
        assert np.all(np.abs(q[m] - real) <= 0.5 + 2e-5)
        assert abs(int(q[m][np.argmax(np.abs(x[m]))])) == 127
        assert abs(float(s[m]) * 127.0 - a) <= 2.0 ** -23 * a
        # dequantisation error within half a step (plus the rounding of 127/a)
        assert np.all(np.abs(q[m] * float(s[m]) - x[m]) <= 0.5 * float(s[m]) * (1 + 1e-4))
    qn, sn = orc.act_quant_i8(-x)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    qs, ss = orc.act_quant_i8(x * np.float32(2.0 ** 7))
    assert np.array_equal(qs, q) and np.array_equal(ss, s * np.float32(2.0 ** 7))
    # ties go to even: with a = 127 the reciprocal is exactly 1
    t = np.array([[127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -126.5]], dtype=np.float32)
    qt, st = orc.act_quant_i8(t)
    assert qt[0].tolist() == [127, 0, 2, 2, 0, -2, -2, 126, -126] and st[0] == np.float32(1.0)


def run_core_pins(orc):
    """The quick pin set used both directly and against planted mutants."""
    rng = np.random.default_rng(7)
    for layout, K, g in [(TENSOR, 1, 0), (TENSOR, 3, 0), (GROUP_F16, 1, 64), (GROUP_F16, 3, 256),
                         (GROUP_F16, 2, 16), (CODEBOOK, 3, 16)]:
        check_dense(orc, layout, K, g, F32, rng=rng)
        check_dense(orc, layout, K, g, BF16, rng=rng)
        check_dense_i8(orc, layout, K, g, rng=rng)
        check_one_hot(orc, layout, K, g if g else 0, rng=rng)
    check_quant(orc, rng)
    check_f16_all(orc)


def check_f16_all(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


# ---------------------------------------------------------------------------
# Tests.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("layout,K,g", CASES)
@pytest.mark.parametrize("x_type", [F32, BF16])
def test_oracle_equals_dense_fake_quant(layout, K, g, x_type):
    check_dense(oracle.default(), layout, K, g, x_type, N=20, Kin=512, M=2)


@pytest.mark.parametrize("layout,K,g", CASES)
def test_oracle_int8_equals_integer_matmul(layout, K, g):
    check_dense_i8(oracle.default(), layout, K, g)


@pytest.mark.parametrize("layout,K,g", [c for c in CASES if c[1] in (1, 3)])
def test_one_hot_reads_one_column(layout, K, g):
    check_one_hot(oracle.default(), layout, K, g)


def test_ragged_shapes_and_edge_sizes():
    orc = oracle.default()
    for (N, Kin, g, M) in [(1, 16, 16, 1), (3, 48, 16, 2), (5, 96, 32, 5), (1, 256, 256, 1),
                           (7, 768, 256, 3)]:
        trits, scales, cb, x = random_problem(2, g, GROUP_F16, N, Kin, M, F32)
        y = orc.gemv_fp(2, g, GROUP_F16, trits, scales, x, F32)
        W = dense_weight(2, g, GROUP_F16, trits, scales, None)
        assert np.allclose(y, x.astype(np.float64) @ W.T, rtol=1e-13, atol=1e-300)
    # empty batch and empty output
    trits, scales, cb, x = random_problem(1, 64, GROUP_F16, 4, 128, 1, F32)
    assert orc.gemv_fp(1, 64, GROUP_F16, trits, scales, x[:0], F32).shape == (0, 4)
    y = orc.gemv_fp(1, 64, GROUP_F16, trits[:, :0], scales[:, :0], x, F32)
    assert y.shape == (1, 0)


def test_constant_planes():
    orc = oracle.default()
    Kin, N = 256, 8
    x = RNG.standard_normal((2, Kin)).astype(np.float32)
    ones = np.full((1, N, Kin), 1, dtype=np.int8)
    unit = np.full((1, N, Kin // 64), 0x3C00, dtype=np.uint16)        # f16 1.0
    y = orc.gemv_fp(1, 64, GROUP_F16, ones, unit, x, F32)
    for m in range(2):
        s = math.fsum(float(v) for v in x[m])
        assert np.allclose(y[m], s, rtol=1e-15, atol=1e-15)
    zeros = np.zeros((3, N, Kin), dtype=np.int8)
    assert np.all(orc.gemv_fp(3, 0, TENSOR, zeros, np.ones(3, np.float32), x, F32) == 0.0)


def test_identity_planes():
    orc = oracle.default()
    n = 64
    x = RNG.standard_normal((1, n)).astype(np.float32)
    s = np.float32(0.0371)
    for sign in (1, -1):
        t = (sign * np.eye(n, dtype=np.int8))[None]
        y = orc.gemv_fp(1, 0, TENSOR, t, np.array([s]), x, F32)[0]
        assert np.array_equal(y, sign * float(s) * x[0].astype(np.float64))


def test_permutations_and_scaling():
    orc = oracle.default()
    K, g, N, Kin = 3, 64, 32, 256
    trits, scales, _, x = random_problem(K, g, GROUP_F16, N, Kin, 2, F32)
    y = orc.gemv_fp(K, g, GROUP_F16, trits, scales, x, F32)
    perm = RNG.permutation(N)
    yp = orc.gemv_fp(K, g, GROUP_F16, trits[:, perm], scales[:, perm], x, F32)
    assert np.array_equal(yp, y[:, perm])
    for e in (-20, 7):
        ys = orc.gemv_fp(K, g, GROUP_F16, trits, scales, x * np.float32(2.0 ** e), F32)
        assert np.array_equal(ys, y * 2.0 ** e)
    assert np.array_equal(orc.gemv_fp(K, g, GROUP_F16, trits, scales, -x, F32), -y)
    # planes add: the K-plane result is the sum of the one-plane results
    parts = sum(orc.gemv_fp(1, g, GROUP_F16, trits[k:k + 1], scales[k:k + 1], x, F32)
                for k in range(K))
    assert np.allclose(parts, y, rtol=1e-14, atol=1e-14)


def test_balanced_ternary_identity():
    levels = sorted({9 * a + 3 * b + c for a in (-1, 0, 1) for b in (-1, 0, 1) for c in (-1, 0, 1)})
    assert levels == list(range(-13, 14)) and len(levels) == 27
    info = json.load(open(os.path.join(GOLDEN, "codec_d3.json")))
    assert info["levels"] == 3 ** info["depth"] == len(levels)
    # information content: 3 trits plus one of 27 codebook symbols per group of 16
    bpw = info["depth"] * math.log2(3) + math.log2(info["scale_codebook_entries"]) / info["group_size"]
    assert f"{bpw:.2f}" == info["bits_per_weight_printed"]
    # the codec scale per plane (3^(K-1-p)) and the card's per-weight level agree
    orc = oracle.default()
    trits, idx, cb, x = random_problem(3, 16, CODEBOOK, 16, 256, 2, F32)
    y = orc.gemv_fp(3, 16, CODEBOOK, trits, idx, x, F32, cb)
    level = 9 * trits[0].astype(np.int64) + 3 * trits[1] + trits[2]
    assert level.min() >= -13 and level.max() <= 13
    W = np.repeat(cb.view(np.float16).astype(np.float64)[idx.astype(np.int64)], 16, axis=1) * level
    assert np.allclose(y, x.astype(np.float64) @ W.T, rtol=1e-14, atol=1e-300)


def test_codebook_recipe():
    cb = gen.codebook_f16(27)
    v = cb.view(np.float16).astype(np.float64)
    assert len(set(cb.tolist())) == 27 and np.all(np.diff(v) > 0)
    assert abs(v[0] - 1e-4) / 1e-4 < 2 ** -10 and abs(v[-1] - 0.1) / 0.1 < 2 ** -10
    ratios = v[1:] / v[:-1]
    assert np.allclose(ratios, 1000.0 ** (1 / 26), rtol=2 ** -9)


def test_bpw_closed_form_matches_page_table():
    table = json.load(open(os.path.join(GOLDEN, "bpw_table.json")))
    for row in table["rows"]:
        K, g = row["K"], row["g"]
        bpw = 2 * K + 16 * K / g
        printed = row["bpw_printed"]
        decimals = len(printed.split(".")[1])
        assert round(bpw, decimals) == float(printed), row


def test_bitnet_shape_inventory_matches_page_sizes():
    info = json.load(open(os.path.join(GOLDEN, "bitnet_2b.json")))
    h, f, L = info["hidden"], info["ffn"], info["layers"]
    kv = info["kv_heads"] * info["head_dim"]
    assert info["query_heads"] * info["head_dim"] == h
    per_layer = 2 * h * h + 2 * kv * h + 3 * f * h
    ternary = L * per_layer
    emb = info["vocab"] * h
    bf16_gb = (ternary + emb) * 2 / 1e9
    assert abs(bf16_gb - info["bf16_size_printed_gb"]) < 0.05
    # 2 bits per ternary weight plus f16 embeddings: consistent with 1.13 GB
    # within the unknown format overhead of the page's binary (a weak pin)
    packed_gb = (ternary / 4 + emb * 2) / 1e9
    assert abs(packed_gb - info["ternary_size_printed_gb"]) / info["ternary_size_printed_gb"] < 0.06


def test_quantiser_properties():
    check_quant(oracle.default())


def test_quantiser_bf16_input_is_its_fp32_value():
    orc = oracle.default()
    xv = RNG.standard_normal((3, 300))
    xb = gen.bf16_bits(xv)
    q1, s1 = orc.act_quant_i8(xb, BF16)
    q2, s2 = orc.act_quant_i8(gen.bf16_bits_to_f32(xb), F32)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


def test_quantiser_clamps_to_127():
    orc = oracle.default()
    # values whose product with fl(127/a) rounds to 127 exactly or just above
    a = np.float32(3.0)
    x = np.array([[a, np.nextafter(a, np.float32(0)), -a, 2.9999998]], dtype=np.float32)
    q, s = orc.act_quant_i8(x)
    assert q.max() <= 127 and q.min() >= -127 and q[0, 0] == 127 and q[0, 2] == -127


def test_f16_decoder_all_patterns():
    check_f16_all(oracle.default())


def test_bf16_decoder_known_values():
    orc = oracle.default()
    known = {0x3F80: 1.0, 0xBF80: -1.0, 0x4049: 3.140625, 0x0000: 0.0, 0xC000: -2.0,
             0x7F80: math.inf, 0x0001: 2.0 ** -133, 0x0080: 2.0 ** -126, 0x3C00: 2.0 ** -7}
    for b, v in known.items():
        assert orc.bf16_to_f32(b) == v, hex(b)
    assert math.copysign(1.0, orc.bf16_to_f32(0x8000)) == -1.0


def test_oracle_rejects_bad_input():
    orc = oracle.default()
    trits, scales, cb, x = random_problem(1, 64, GROUP_F16, 4, 128, 1, F32)
    bad = trits.copy()
    bad[0, 0, 0] = 2
    with pytest.raises(oracle.OracleError):
        orc.gemv_fp(1, 64, GROUP_F16, bad, scales, x, F32)
    with pytest.raises(oracle.OracleError):
        orc.gemv_fp(1, 48, GROUP_F16, trits, scales, x, F32)      # Kin % g != 0
    xn = x.copy()
    xn[0, 3] = np.nan
    with pytest.raises(oracle.OracleError):
        orc.gemv_fp(1, 64, GROUP_F16, trits, scales, xn, F32)
    t3, idx, cb, x3 = random_problem(3, 16, CODEBOOK, 4, 64, 1, F32)
    idx = idx.copy()
    idx[0, 0] = 27
    with pytest.raises(oracle.OracleError):
        orc.gemv_fp(3, 16, CODEBOOK, t3, idx, x3, F32, cb)


def test_core_pins_pass_on_the_oracle():
    run_core_pins(oracle.default())


# Each entry plants one plausible mistake in a copy of oracle.c.
MUTANTS = [
    ("wrong sign for -1", "else if (t == -1) p -= xv;", "else if (t == -1) p += xv;"),
    ("dropped last plane", "for (k = 0; k < K; ++k) {\n                int64_t grp;\n                for (grp = 0; grp < G; ++grp) {\n                    double p",
     "for (k = 0; k < K - 1; ++k) {\n                int64_t grp;\n                for (grp = 0; grp < G; ++grp) {\n                    double p"),
    ("transposed scale index", "((int64_t)k * N + n) * G + grp", "((int64_t)n * K + k) * G + grp"),
    ("codebook weight reversed", "for (j = 0; j < K - 1 - k; ++j) w *= 3.0;", "for (j = 0; j < k; ++j) w *= 3.0;"),
    ("group shifted by one column", "for (j = grp * gs; j < (grp + 1) * gs && j < Kin; ++j) {\n                        int8_t t = trits[((int64_t)k * N + n) * Kin + j];\n                        double",
     "for (j = grp * gs + 1; j < (grp + 1) * gs + 1 && j < Kin; ++j) {\n                        int8_t t = trits[((int64_t)k * N + n) * Kin + j];\n                        double"),
    ("ties away from zero", "float r = rintf(v * inv);", "float r = roundf(v * inv);"),
    ("f16 exponent bias", "exp - 25", "exp - 24"),
    ("int8 sign", "else if (t == -1) p -= xv;\n                    }\n                    total",
     "else if (t == -1) p += xv;\n                    }\n                    total"),
    ("epilogue rounding order", "y32[m * N + n] = (float)total * c;",
     "y32[m * N + n] = (float)((double)total * (double)((const float*)scales)[0] * (double)xs[m]) + 0.0f * c;"),
    ("x row stride", "x_value(x_type, x, m * Kin + j)", "x_value(x_type, x, m + j)"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new, tmp_path):
    src = open(oracle.SRC).read()
    assert old in src, "mutation anchor missing: " + name
    mutated = src.replace(old, new, 1)
    csrc = tmp_path / "oracle_mutant.c"
    csrc.write_text(mutated)
    so = tmp_path / "liboracle_mutant.so"
    subprocess.check_call(["gcc", *oracle._CFLAGS, str(csrc), "-o", str(so), "-lm"])
    orc = oracle.Oracle(str(so))
    with pytest.raises(AssertionError):
        run_core_pins(orc)
