"""The seeded input generator (host side, no GPU)."""
from __future__ import annotations

import numpy as np

from synth import gen, inputs
from synth.configs import CASES, GROUP_F16


def test_splitmix64_published_first_output():
    # SplitMix64 started from state 0 first returns 0xE220A8397B1DCDAF.
    assert int(gen.stream(0, 0, 1)[0]) == 0xE220A8397B1DCDAF
    assert gen.mix64_int(gen.GAMMA) == 0xE220A8397B1DCDAF


def test_stream_is_counter_based():
    full = gen.stream(12345, 0, 1000)
    assert np.array_equal(gen.stream(12345, 317, 100), full[317:417])
    assert len(set(full.tolist())) == 1000


def test_elementary_functions_accuracy():
    x = np.linspace(2.0 ** -53, 1.0, 200001)
    assert np.max(np.abs(gen.det_ln(x) - np.log(x)) / np.maximum(1, np.abs(np.log(x)))) < 1e-15
    u = np.linspace(0, 1, 200001, endpoint=False)
    assert np.max(np.abs(gen.det_cos2pi(u) - np.cos(2 * np.pi * u))) < 1e-15
    y = np.linspace(0, 80, 200001)
    r = gen.det_sqrt(y)
    assert r[0] == 0.0 and np.max(np.abs(r[1:] - np.sqrt(y[1:])) / np.sqrt(y[1:])) < 4e-16
    z = np.linspace(-25, 5, 200001)
    assert np.max(np.abs(gen.det_exp(z) - np.exp(z)) / np.exp(z)) < 1e-15


def test_distributions():
    n = gen.normal(99, 0, 400000)
    assert abs(n.mean()) < 0.01 and abs(n.std() - 1) < 0.01
    t = gen.trits(5, 0, 400000)
    fr = [(t == v).mean() for v in (-1, 0, 1)]
    assert abs(fr[0] - 0.3) < 0.005 and abs(fr[1] - 0.4) < 0.005 and abs(fr[2] - 0.3) < 0.005
    d = gen.digits(6, 0, 300000)
    assert all(abs((d == v).mean() - 1 / 3) < 0.005 for v in (-1, 0, 1))
    i = gen.indices(7, 0, 270000, 27)
    assert i.min() == 0 and i.max() == 26 and np.all(np.bincount(i, minlength=27) > 9000)
    lu = gen.log_uniform(8, 0, 200000, 1e-3, 1e-1)
    assert lu.min() >= 1e-3 and lu.max() <= 1e-1 and abs(np.log10(lu).mean() + 2) < 0.01


def test_bf16_round_to_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5], np.float32)
    b = gen.f32_to_bf16_bits(f)
    assert b.tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020]
    assert np.array_equal(gen.bf16_bits_to_f32(b)[[0, 4]], np.array([1.0, -2.5], np.float32))


def test_row_subsets_match_full_tensor():
    case = CASES["cfg3"]
    full = inputs.projection(case, 2, 4, 64, 512)
    rows = [0, 5, 63]
    part = inputs.projection(case, 2, 4, 64, 512, rows=rows)
    assert np.array_equal(part["trits"], full["trits"][:, rows])
    assert np.array_equal(part["scales"], full["scales"][:, rows])
    assert np.array_equal(part["x"], full["x"])
    case4 = CASES["cfg4"]
    f4 = inputs.projection(case4, 1, 1, 32, 256)
    p4 = inputs.projection(case4, 1, 1, 32, 256, rows=[3, 31])
    assert np.array_equal(p4["trits"], f4["trits"][:, [3, 31]])
    assert np.array_equal(p4["scales"], f4["scales"][[3, 31]])


def test_case_recipes():
    c1 = inputs.projection(CASES["cfg1"], 0, 0, 256, 512)
    assert c1["trits"].shape == (1, 256, 512) and c1["scales"].shape == (1, 256, 8)
    assert c1["x"].dtype == np.float32 and c1["x"].shape == (1, 512)
    s = c1["scales"].view(np.float16).astype(np.float64)
    assert s.min() >= 1e-3 * (1 - 2 ** -10) and s.max() <= 1e-1 * (1 + 2 ** -10)
    c3 = inputs.projection(CASES["cfg3"], 0, 1, 64, 512)
    sc = c3["scales"].view(np.float16).astype(np.float64)
    # plane k is drawn from [1e-3, 1e-1] * 3^-k
    for k in range(3):
        assert sc[k].max() <= 0.1 / 3 ** k * (1 + 2 ** -10)
    assert c3["x"].dtype == np.uint16
    c2 = inputs.projection(CASES["cfg2"], 3, 6, 64, 256)
    assert c2["scales"].dtype == np.float32 and c2["scales"].shape == (1,)
    assert CASES["cfg3"].layout == GROUP_F16


def test_routing_shapes():
    """Each token has top_k distinct experts; each expert's rows are its tokens."""
    from synth.configs import MOES
    moe = MOES["moe_small"]
    for layer in range(moe.layers):
        route = inputs.moe_routing(moe, layer)
        assert route.shape == (moe.batch, moe.top_k)
        assert all(len(set(r)) == moe.top_k for r in route)
        rows = inputs.moe_expert_rows(moe, layer)
        assert sum(len(t) for t, _ in rows) == moe.batch * moe.top_k
        for e, (toks, pairs) in enumerate(rows):
            for t, pr in zip(toks, pairs):
                assert route[t][pr - t * moe.top_k] == e
