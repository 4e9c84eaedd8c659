"""Pins of the ternarizer part of the CPU oracle (no GPU).

oracle_ternarize fits a dense weight into K per-group-scaled trit planes
(greedy residual; per plane the absmean threshold, then the least-squares
scale of that plane) or into the balanced-ternary codec (uniform levels, a
scale from the codebook per group of 16).  Held to:
  * the f16 rounding against numpy's float16 (a library routine);
  * the defining property of the greedy planes: no plane increases any
    group's squared error (its scale is optimal for it), so the error never
    grows with K; the scale equals the least-squares optimum <R, t> / <t, t>
    computed by numpy; a weight that is exactly s * t (t = +-1) is
    recovered exactly by one plane and leaves zero planes after it;
  * closed forms (a constant row, a ramp);
  * the codec on its own grid (w = cb[i] q, max |q| = 13) recovered exactly
    with the card's digit weights 9, 3, 1; its error bound cb[idx] / 2;
    the smallest adequate codebook entry;
  * the fitted weight reproduced by the pinned product oracle (gemv_fp);
and a mutation check plants typical mistakes in a copy of oracle.c.
"""
from __future__ import annotations

import subprocess

import numpy as np
import pytest

import oracle
from oracle import CODEBOOK, F32, GROUP_F16, TENSOR
from synth import gen

RNG = np.random.default_rng(31)
CB = gen.codebook_f16(27)


def f16(v):
    return np.asarray(v, dtype=np.uint16).view(np.float16).astype(np.float64)


def dequant(K, g, layout, trits, scales, codebook=None):
    """fp64 sum of the scaled planes, [K][N][Kin] partial sums."""
    _, N, Kin = trits.shape
    out = np.zeros((K, N, Kin))
    for k in range(K):
        if layout == TENSOR:
            s = np.full((N, Kin), float(scales[k]))
        elif layout == GROUP_F16:
            s = np.repeat(f16(scales[k]), g, axis=1)
        else:
            s = np.repeat(f16(codebook)[scales.astype(np.int64)], g, axis=1) * 3.0 ** (K - 1 - k)
        out[k] = s * trits[k]
    return np.cumsum(out, axis=0)


def run_ternarize_pins(orc):
    # f16 rounding = numpy's (ties to even), inside the finite range
    vals = np.concatenate([RNG.standard_normal(4000) * 10.0 ** RNG.integers(-8, 4, 4000),
                           [0.0, 65504.0, 65519.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 1.0 + 2.0 ** -11,
                            1.0 + 3 * 2.0 ** -11, 6.1e-5]]).astype(np.float32)
    vals = vals[np.abs(vals) < 65520.0]
    want = vals.astype(np.float16).view(np.uint16)
    got = np.array([orc.f32_to_f16(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, want)
    assert orc.f32_to_f16(1e6) == 0x7BFF and orc.f32_to_f16(-1e6) == 0xFBFF   # saturates

    for layout, g in ((GROUP_F16, 16), (GROUP_F16, 64), (TENSOR, 0)):
        w = (RNG.standard_normal((12, 128)) * 0.05).astype(np.float32)
        trits, scales = orc.ternarize(4, g, layout, w)
        assert set(np.unique(trits)) <= {-1, 0, 1}
        rec = dequant(4, g, layout, trits, scales)
        res = w.astype(np.float64)[None] - rec
        gs = 128 if layout == TENSOR else g
        prev = w.astype(np.float64)
        for k in range(4):
            # the plane's scale is the least-squares one for its trits (to f16 / fp32 rounding)
            tk = trits[k].astype(np.float64).reshape(12 * 128 // gs if layout != TENSOR else 1, -1)
            pr = prev.reshape(tk.shape)
            nz = np.maximum((tk != 0).sum(axis=1), 1)
            ls = (pr * tk).sum(axis=1) / nz
            sk = (np.repeat(f16(scales[k]), 1) if layout == GROUP_F16 else np.array([float(scales[k])])).reshape(-1)
            assert np.allclose(sk, ls, rtol=2e-3, atol=1e-12), (layout, k)
            # no group's squared error grows
            e_prev = (pr ** 2).sum(axis=1)
            e_new = (res[k].reshape(tk.shape) ** 2).sum(axis=1)
            assert np.all(e_new <= e_prev * (1 + 1e-9) + 1e-18), (layout, k)
            prev = res[k]
        err = np.sqrt(np.sum(res ** 2, axis=(1, 2)))
        assert np.all(np.diff(err) <= 1e-9) and err[-1] < 0.15 * np.sqrt(np.sum(w.astype(np.float64) ** 2))
        # the planes reproduce through the product oracle: gemv_fp of the fit = dequantised W @ x
        x = RNG.standard_normal((2, 128)).astype(np.float32)
        y = orc.gemv_fp(4, g, layout, trits, scales, x, F32)
        assert np.allclose(y, x.astype(np.float64) @ rec[-1].T, rtol=1e-12, atol=1e-12)

    # on-grid: w = s t with t = +-1 and s an f16 value, per group
    s_bits = gen.f16_bits(RNG.uniform(0.01, 0.1, (6, 4)))
    t = np.where(RNG.random((6, 64)) < 0.5, -1, 1).astype(np.int8)
    w = (np.repeat(f16(s_bits), 16, axis=1) * t).astype(np.float32)
    trits, scales = orc.ternarize(3, 16, GROUP_F16, w)
    assert np.array_equal(trits[0], t) and np.array_equal(scales[0], s_bits)
    assert not trits[1:].any() and not scales[1:].any()
    # closed forms: a constant row c gives t = 1, s = c; the ramp 1..16 has
    # absmean 8.5, so 1..4 round to 0 and s is the mean of 5..16, 10.5
    w = np.zeros((2, 16), dtype=np.float32)
    w[0] = 0.75
    w[1] = np.arange(1, 17, dtype=np.float32)
    trits, scales = orc.ternarize(1, 16, GROUP_F16, w)
    assert f16(scales[0, 0, 0]) == 0.75 and f16(scales[0, 1, 0]) == 10.5
    assert list(trits[0, 0]) == [1] * 16 and list(trits[0, 1]) == [0, 0, 0, 0] + [1] * 12
    trits, scales = orc.ternarize(1, 0, TENSOR, w)
    # whole tensor: absmean (12 + 136) / 32 = 4.625, so row 0 and 1, 2 fall
    # below 2.3125; s is the mean of 3..16, 133 / 14 = 9.5
    assert not trits[0, 0].any() and list(trits[0, 1]) == [0, 0] + [1] * 14
    assert scales[0] == np.float32(9.5)

    # the codec: on its grid, exact; the card's levels 9 t2 + 3 t1 + t0
    cbv = f16(CB)
    idx = RNG.integers(0, 27, (5, 8))
    q = RNG.integers(-13, 14, (5, 128))
    q[:, ::16] = 13 * np.where(RNG.random((5, 8)) < 0.5, -1, 1)   # every group reaches 13
    w = (np.repeat(cbv[idx], 16, axis=1) * q).astype(np.float32)
    assert np.array_equal(w.astype(np.float64), np.repeat(cbv[idx], 16, axis=1) * q)
    trits, scales = orc.ternarize(3, 16, CODEBOOK, w, CB)
    assert np.array_equal(scales, idx)
    assert np.array_equal(9 * trits[0].astype(int) + 3 * trits[1] + trits[2], q)
    # off the grid: the smallest entry >= max|w| / 13, error <= cb[idx] / 2
    w = (RNG.standard_normal((8, 256)) * 0.02).astype(np.float32)
    trits, scales = orc.ternarize(3, 16, CODEBOOK, w, CB)
    lev = 9 * trits[0].astype(int) + 3 * trits[1] + trits[2]
    s = cbv[scales.astype(np.int64)]
    amax = np.abs(w).reshape(8, 16, 16).max(axis=2) / np.float32(13)
    assert np.all(s >= amax) and np.all(np.where(scales > 0, cbv[np.maximum(scales.astype(np.int64) - 1, 0)] < amax, True))
    assert np.all(np.abs(w - np.repeat(s, 16, axis=1) * lev) <= np.repeat(s, 16, axis=1) / 2 + 1e-12)


def test_ternarize_pins_pass_on_the_oracle():
    run_ternarize_pins(oracle.default())


def test_ternarize_rejects_bad_input():
    orc = oracle.default()
    w = np.zeros((4, 64), dtype=np.float32)
    w[1, 3] = np.inf
    with pytest.raises(oracle.OracleError):
        orc.ternarize(2, 16, GROUP_F16, w)
    with pytest.raises(oracle.OracleError):
        orc.ternarize(3, 16, CODEBOOK, np.zeros((4, 64), np.float32), CB[::-1].copy())   # descending


TERNARIZE_MUTANTS = [
    ("absmax threshold", "for (i = grp * gs; i < (grp + 1) * gs; ++i) sum += fabs((double)R[n * Kin + i]);",
     "for (i = grp * gs; i < (grp + 1) * gs; ++i) sum = fmax(sum, fabs((double)R[n * Kin + i]) * (double)gs);"),
    ("threshold at the absmean", "if (a > 0.0f && fabsf(R[n * Kin + i]) > 0.5f * a) t",
     "if (a > 0.0f && fabsf(R[n * Kin + i]) > 1.0f * a) t"),
    ("absmean kept as the scale", "sc = nz > 0 ? (float)(sum_nz / (double)nz) : 0.0f;\n                    {",
     "sc = a;\n                    {"),
    ("no residual update", "R[n * Kin + i] = R[n * Kin + i] - sc * (float)trits[((int64_t)k * N + n) * Kin + i];",
     "(void)0;"),
    ("f16 ties away", "q = nearbyint((m - 1.0) * 1024.0);", "q = floor((m - 1.0) * 1024.0 + 0.5);"),
    ("codec digit order", "trits[((int64_t)p * N + n) * Kin + i] = dig[K - 1 - p];",
     "trits[((int64_t)p * N + n) * Kin + i] = dig[p];"),
    ("codec largest entry", "idx = j;\n                        break;", "idx = j;"),
    ("codec levels", "const int L = (K == 1) ? 1 : (K == 2 ? 4 : (K == 3 ? 13 : 40));",
     "const int L = (K == 1) ? 1 : (K == 2 ? 4 : (K == 3 ? 12 : 40));"),
]


@pytest.mark.parametrize("name,old,new", TERNARIZE_MUTANTS, ids=[m[0] for m in TERNARIZE_MUTANTS])
def test_planted_ternarize_mistake_is_caught(name, old, new, tmp_path):
    src = open(oracle.SRC).read()
    assert old in src, "mutation anchor missing: " + name
    csrc = tmp_path / "oracle_mutant.c"
    csrc.write_text(src.replace(old, new, 1))
    so = tmp_path / "liboracle_mutant.so"
    subprocess.check_call(["gcc", *oracle._CFLAGS, str(csrc), "-o", str(so), "-lm"])
    with pytest.raises(AssertionError):
        run_ternarize_pins(oracle.Oracle(str(so)))
