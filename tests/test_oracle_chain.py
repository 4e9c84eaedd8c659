"""Pins of the decode-chain part of the CPU oracle (no GPU).

The chain runs BitNet b1.58 layers as the QORA-LLM-2B page's "SubLN
Pattern" listing does, for one token at position 0 (oracle.c,
oracle_bitnet_layer).  Its pieces and its wiring are held to:
  * RMSNorm closed forms and invariants: a one-hot input, power-of-two
    scaling, odd symmetry, unit mean square, and an input whose sum of
    squares fp32 accumulation would round away;
  * the squared ReLU on special values;
  * an independent composition of the layer in numpy: numpy's integer
    matmul for the ternary products, a real softmax attention over the one
    cached key for the attention step, numpy float32 for the residuals and
    the squared-ReLU product;
  * the residual path with zero weights, and a dense fp64 forward pass with
    unquantised activations (loose);
and a mutation check plants typical wiring mistakes in a copy of oracle.c and
requires each to fail at least one pin.
"""
from __future__ import annotations

import math
import subprocess

import numpy as np
import pytest

import oracle
from synth import inputs
from synth.configs import CHAINS

SMALL = CHAINS["chain_small"]


def small_layer(chain=SMALL, layer=0):
    ws = [inputs.chain_projection(chain, layer, p) for p in range(7)]
    trits = [w["trits"][0] for w in ws]
    s_w = np.array([w["scales"][0] for w in ws], dtype=np.float32)
    norms = [inputs.chain_norm(chain, layer, i) for i in range(4)]
    return trits, s_w, norms


# ---------------------------------------------------------------------------
# Independent formulations.
# ---------------------------------------------------------------------------
def linear_matmul(orc, t, s_w, x):
    """One ternary linear on the int8 quantisation of x, with numpy's int64 matmul."""
    q, s = orc.act_quant_i8(x.reshape(1, -1))
    acc = t.astype(np.int64) @ q[0].astype(np.int64)
    c = np.float32(s_w) * s[0]
    return acc.astype(np.float32) * c


def attention_one_key(q, k, v, n_heads, n_kv, hd):
    """Softmax attention of every query head over the single cached key of
    its KV group (grouped-query attention, KV head j serving query heads
    j * n_rep .. (j + 1) * n_rep - 1)."""
    n_rep = n_heads // n_kv
    out = np.empty(n_heads * hd, dtype=np.float32)
    for h in range(n_heads):
        j = h // n_rep
        qh, kj, vj = q[h * hd:(h + 1) * hd], k[j * hd:(j + 1) * hd], v[j * hd:(j + 1) * hd]
        scores = np.array([np.dot(qh.astype(np.float64), kj.astype(np.float64)) / math.sqrt(hd)])
        p = np.exp(scores - scores.max())
        p /= p.sum()
        out[h * hd:(h + 1) * hd] = (p[0] * vj.astype(np.float64)).astype(np.float32)
    return out


def compose_layer(orc, chain, trits, s_w, norms, x):
    hidden, inter, nh, nkv, hd, eps = chain.dims()
    f32 = np.float32
    h = orc.rms_norm(x, norms[0], eps)
    q = linear_matmul(orc, trits[0], s_w[0], h)
    k = linear_matmul(orc, trits[1], s_w[1], h)
    v = linear_matmul(orc, trits[2], s_w[2], h)
    a = orc.rms_norm(attention_one_key(q, k, v, nh, nkv, hd), norms[1], eps)
    x1 = (x + linear_matmul(orc, trits[3], s_w[3], a)).astype(f32)
    h2 = orc.rms_norm(x1, norms[2], eps)
    g = linear_matmul(orc, trits[4], s_w[4], h2)
    u = linear_matmul(orc, trits[5], s_w[5], h2)
    gp = np.maximum(g, f32(0))
    f = orc.rms_norm((gp * gp) * u, norms[3], eps)
    x2 = (x1 + linear_matmul(orc, trits[6], s_w[6], f)).astype(f32)
    return x2, np.concatenate([q, k, v])


def dense_layer_f64(chain, trits, s_w, norms, x):
    """The listing in fp64 with unquantised activations and dequantised weights."""
    hidden, inter, nh, nkv, hd, eps = chain.dims()
    W = [t.astype(np.float64) * float(s) for t, s in zip(trits, s_w)]
    nw = [n.astype(np.float64) for n in norms]

    def rms(z, w):
        return z / np.sqrt(np.mean(z * z) + eps) * w
    x = x.astype(np.float64)
    h = rms(x, nw[0])
    v = W[2] @ h
    rep = nh // nkv
    a = np.concatenate([v[(hh // rep) * hd:(hh // rep + 1) * hd] for hh in range(nh)])
    x1 = x + W[3] @ rms(a, nw[1])
    h2 = rms(x1, nw[2])
    f = np.maximum(W[4] @ h2, 0.0) ** 2 * (W[5] @ h2)
    return x1 + W[6] @ rms(f, nw[3])


# ---------------------------------------------------------------------------
def run_chain_pins(orc):
    rng = np.random.default_rng(7)
    # RMSNorm, one-hot: with eps = 0 and n = 256 the mean square is a^2 / 256,
    # so out_j = sign(a) * 16 * w_j exactly and every other entry is 0
    n = 256
    w = (0.5 + rng.random(n)).astype(np.float32)
    for a, j in ((2.0 ** 5, 3), (-(2.0 ** -9), 200)):
        x = np.zeros(n, dtype=np.float32)
        x[j] = a
        out = orc.rms_norm(x, w, 0.0)
        exp = np.zeros(n, dtype=np.float32)
        exp[j] = np.float32(math.copysign(16.0, a)) * w[j]
        assert np.array_equal(out, exp)
    # power-of-two scaling leaves the result unchanged (eps = 0); odd symmetry
    x = rng.standard_normal(1000).astype(np.float32)
    w = (0.5 + rng.random(1000)).astype(np.float32)
    base = orc.rms_norm(x, w, 0.0)
    for e in (-7, 5):
        assert np.array_equal(orc.rms_norm(x * np.float32(2.0 ** e), w, 0.0), base)
    assert np.array_equal(orc.rms_norm(-x, w, 1e-5), -orc.rms_norm(x, w, 1e-5))
    # unit mean square with unit weights
    assert abs(float(np.mean(orc.rms_norm(x, np.ones_like(x), 0.0).astype(np.float64) ** 2)) - 1.0) < 1e-6
    # the sum of squares keeps the small terms: 2^24 + 4096 * 0.25 (fp32
    # accumulation would stop at 2^24, moving the result by ~256 ulp)
    x = np.full(4097, 0.5, dtype=np.float32)
    x[0] = 4096.0
    exact = 4096.0 / math.sqrt((2.0 ** 24 + 1024.0) / 4097.0)
    got = float(orc.rms_norm(x, np.ones_like(x), 0.0)[0])
    assert abs(got - exact) <= 2 * np.spacing(np.float32(exact))
    # squared ReLU times up
    g = np.array([-3.0, 0.0, 2.0, 0.5, -0.0], dtype=np.float32)
    u = np.array([7.0, -2.0, 3.0, -8.0, 1.0], dtype=np.float32)
    assert np.array_equal(orc.relu2_mul(g, u), np.array([0.0, 0.0, 12.0, -2.0, 0.0], dtype=np.float32))

    # the layer against the independent composition, bit for bit, two layers
    x = inputs.chain_input(SMALL)
    for layer in range(2):
        trits, s_w, norms = small_layer(SMALL, layer)
        want, want_qkv = compose_layer(orc, SMALL, trits, s_w, norms, x)
        got, got_qkv = orc.bitnet_layer(SMALL.dims(), trits, s_w, norms, x)
        assert np.array_equal(got_qkv, want_qkv)
        assert np.array_equal(got, want)
        # and near the dense fp64 pass: the int8 activations (steps of
        # absmax / 127, heavy-tailed after the squared ReLU) move the layer's
        # update by ~6% of its rms here; a wiring mistake moves it by O(1)
        dense = dense_layer_f64(SMALL, trits, s_w, norms, x)
        delta = dense - x
        assert np.max(np.abs(got - dense)) <= 0.15 * np.sqrt(np.mean(delta * delta))
        x = got
    # zero o and down weights: the residual stream passes through unchanged
    trits, s_w, norms = small_layer(SMALL, 0)
    x0 = inputs.chain_input(SMALL)
    zt = [t if p not in (3, 6) else np.zeros_like(t) for p, t in enumerate(trits)]
    got, _ = orc.bitnet_layer(SMALL.dims(), zt, s_w, norms, x0)
    assert np.array_equal(got, x0)


def test_chain_pins_pass_on_the_oracle():
    run_chain_pins(oracle.default())


def test_small_chain_reaches_every_layer():
    """Six layers in a row stay finite and keep changing the state."""
    orc = oracle.default()
    x = inputs.chain_input(SMALL)
    for layer in range(SMALL.layers):
        trits, s_w, norms = small_layer(SMALL, layer)
        nx, _ = orc.bitnet_layer(SMALL.dims(), trits, s_w, norms, x)
        assert np.all(np.isfinite(nx)) and not np.array_equal(nx, x)
        x = nx


def test_bitnet_chain_weights_are_the_decode_stack():
    """The BitNet chain draws exactly the decode stack's projections."""
    from synth.configs import CASES
    chain = CHAINS["chain"]
    for layer, p in ((0, 1), (29, 2)):
        _, N, Kin = chain.proj_shapes()[p]
        a = inputs.chain_projection(chain, layer, p)
        b = inputs.projection(CASES["cfg2"], layer, p, N, Kin)
        assert np.array_equal(a["trits"], b["trits"]) and np.array_equal(a["scales"], b["scales"])


def test_layer_rejects_bad_shapes():
    orc = oracle.default()
    trits, s_w, norms = small_layer()
    hidden, inter, nh, nkv, hd, eps = SMALL.dims()
    with pytest.raises(oracle.OracleError):
        orc.bitnet_layer((hidden, inter, nh, 3, hd, eps), trits, s_w, norms, inputs.chain_input(SMALL))


CHAIN_MUTANTS = [
    ("plain relu", "out[i] = (a * a) * u[i];", "out[i] = a * u[i];"),
    ("interleaved kv heads", "kvh = head / (n_heads / n_kv);", "kvh = head % n_kv;"),
    ("attention-sub norm with the input weight", "oracle_rms_norm(nq, a, w_attn_sub, eps, a)",
     "oracle_rms_norm(nq, a, w_in, eps, a)"),
    ("residual from the normed state", "x1[i] = x[i] + o[i];", "x1[i] = h[i] + o[i];"),
    ("no FFN-sub norm", "if ((rc = oracle_rms_norm(inter, f, w_ffn_sub, eps, f))) goto done;", ""),
    ("fp32 sum of squares", "double ss = 0.0;", "float ss = 0.0f;"),
    ("eps outside the root", "r = 1.0f / sqrtf(ms + eps);", "r = 1.0f / sqrtf(ms) + eps;"),
    ("gate and up swapped", "linear_i8(inter, hidden, trits[4], s_w[4], h, g, qt)",
     "linear_i8(inter, hidden, trits[5], s_w[5], h, g, qt)"),
]


@pytest.mark.parametrize("name,old,new", CHAIN_MUTANTS, ids=[m[0] for m in CHAIN_MUTANTS])
def test_planted_chain_mistake_is_caught(name, old, new, tmp_path):
    src = open(oracle.SRC).read()
    assert old in src, "mutation anchor missing: " + name
    csrc = tmp_path / "oracle_mutant.c"
    csrc.write_text(src.replace(old, new, 1))
    so = tmp_path / "liboracle_mutant.so"
    subprocess.check_call(["gcc", *oracle._CFLAGS, str(csrc), "-o", str(so), "-lm"])
    with pytest.raises(AssertionError):
        run_chain_pins(oracle.Oracle(str(so)))
