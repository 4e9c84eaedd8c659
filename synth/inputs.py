"""Canonical host-side inputs of one projection of a workload.

Canonical layouts (the ones the C ABI's pack call and the oracle take):
  trits     int8  [K][N][Kin]   values in {-1, 0, +1} (digits for the codec)
  TENSOR    fp32  [K]           one scale per plane
  GROUP_F16 u16   [K][N][G]     f16 bits, G = Kin / g
  CODEBOOK  u8    [N][G]        index into an f16 codebook (u16 bits [n_cb])
  x         fp32 or bf16 bits   [M][Kin]

Value recipes, as the workloads state them or, where they are silent, the
plainest reading that the rest supports:
  trits     P(-1) = P(+1) = 0.3, P(0) = 0.4
  digits    uniform over {-1, 0, +1}
  TENSOR    log-uniform [1e-3, 1e-1], one draw per plane, rounded to fp32
  GROUP_F16 log-uniform [1e-3, 1e-1] times 3^-k for plane k, rounded to f16
  CODEBOOK  index uniform over 0..26; codebook log-spaced [1e-4, 1e-1]
  x         N(0, 1), rounded to fp32, or fp32 then bf16

Because every draw is counter based, ``rows`` selects a subset of output rows
and produces exactly the values the full tensor holds at those rows.
"""
from __future__ import annotations

import numpy as np

from . import gen
from .configs import (BF16, CODEBOOK, F32, GROUP_F16, I8, KIND_DIGITS, KIND_DENSE, KIND_INDEX,
                      KIND_NORM, KIND_ROUTE, KIND_SCALES, KIND_TRITS, KIND_X, TENSOR)

N_CODEBOOK = 27


def _rows_of(n: int, rows):
    return np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)


def plane_values(seed: int, K: int, N: int, Kin: int, rows=None, digit=False) -> np.ndarray:
    """int8 [K][len(rows)][Kin] slice of the [K][N][Kin] trit (or digit) tensor."""
    rows = _rows_of(N, rows)
    draw = gen.digits if digit else gen.trits
    out = np.empty((K, len(rows), Kin), dtype=np.int8)
    for k in range(K):
        for j, n in enumerate(rows):
            out[k, j] = draw(seed, (k * N + int(n)) * Kin, Kin)
    return out


def plane_values_full(seed: int, K: int, N: int, Kin: int, digit=False) -> np.ndarray:
    draw = gen.digits if digit else gen.trits
    return draw(seed, 0, K * N * Kin).reshape(K, N, Kin)


def group_scales(seed: int, K: int, N: int, G: int, rows=None) -> np.ndarray:
    """u16 f16 bits [K][len(rows)][G]: log-uniform [1e-3, 1e-1] * 3^-k."""
    rows = _rows_of(N, rows)
    out = np.empty((K, len(rows), G), dtype=np.uint16)
    for k in range(K):
        div = float(3 ** k)
        if rows is None or len(rows) == N:
            v = gen.log_uniform(seed, k * N * G, N * G, 1e-3, 1e-1) / div
            out[k] = gen.f16_bits(v).reshape(N, G)[rows]
        else:
            for j, n in enumerate(rows):
                v = gen.log_uniform(seed, (k * N + int(n)) * G, G, 1e-3, 1e-1) / div
                out[k, j] = gen.f16_bits(v)
    return out


def tensor_scales(seed: int, K: int) -> np.ndarray:
    """fp32 [K]: log-uniform [1e-3, 1e-1], one per plane."""
    return gen.log_uniform(seed, 0, K, 1e-3, 1e-1).astype(np.float32)


def codebook_indices(seed: int, N: int, G: int, rows=None) -> np.ndarray:
    rows = _rows_of(N, rows)
    out = np.empty((len(rows), G), dtype=np.uint8)
    for j, n in enumerate(rows):
        out[j] = gen.indices(seed, int(n) * G, G, N_CODEBOOK)
    return out


def activations(seed: int, M: int, Kin: int, x_type: int) -> np.ndarray:
    """x [M][Kin]: fp32 values, or bf16 bits (u16) for BF16."""
    v = gen.normal(seed, 0, M * Kin).reshape(M, Kin)
    if x_type == BF16:
        return gen.bf16_bits(v)
    return v.astype(np.float32)


def seeds(cfg: int, layer: int, proj: int) -> dict:
    return {
        "trits": gen.tensor_seed(cfg, layer, proj, KIND_TRITS),
        "digits": gen.tensor_seed(cfg, layer, proj, KIND_DIGITS),
        "scales": gen.tensor_seed(cfg, layer, proj, KIND_SCALES),
        "index": gen.tensor_seed(cfg, layer, proj, KIND_INDEX),
        "x": gen.tensor_seed(cfg, layer, proj, KIND_X),
    }


def projection(case, layer: int, proj: int, N: int, Kin: int, rows=None, M=None) -> dict:
    """All canonical inputs of one projection (optionally only some rows)."""
    s = seeds(case.cfg, layer, proj)
    K, g = case.planes, case.group
    M = case.M if M is None else M
    d = {"K": K, "g": g, "layout": case.layout, "N": N, "Kin": Kin, "M": M,
         "x_type": case.x_type, "rows": rows}
    if case.layout == CODEBOOK:
        d["trits"] = plane_values(s["digits"], K, N, Kin, rows, digit=True) if rows is not None \
            else plane_values_full(s["digits"], K, N, Kin, digit=True)
        d["scales"] = codebook_indices(s["index"], N, Kin // g, rows)
        d["codebook"] = gen.codebook_f16(N_CODEBOOK)
    else:
        d["trits"] = plane_values(s["trits"], K, N, Kin, rows) if rows is not None \
            else plane_values_full(s["trits"], K, N, Kin)
        if case.layout == GROUP_F16:
            d["scales"] = group_scales(s["scales"], K, N, Kin // g, rows)
        else:
            d["scales"] = tensor_scales(s["scales"], K)
        d["codebook"] = None
    xt = F32 if case.x_type in (F32, I8) else BF16
    d["x"] = activations(s["x"], M, Kin, xt)
    return d


def chain_projection(chain, layer: int, proj: int) -> dict:
    """Projection ``proj`` (q, k, v, o, gate, up, down) of a chain layer:
    trits int8 [1][N][Kin] and the per-tensor scale fp32 [1], drawn as the
    BitNet decode stack draws them (its seeds when weights_cfg is 2)."""
    _, N, Kin = chain.proj_shapes()[proj]
    s = seeds(chain.weights_cfg, layer, proj)
    return {"trits": plane_values_full(s["trits"], 1, N, Kin), "scales": tensor_scales(s["scales"], 1),
            "N": N, "Kin": Kin}


def chain_norm(chain, layer: int, which: int) -> np.ndarray:
    """RMSNorm weight ``which`` (0 input, 1 attention-sub, 2 post-attention,
    3 FFN-sub) of a chain layer: fp32 uniform over [0.5, 1.5)."""
    n = chain.norm_sizes()[which]
    seed = gen.tensor_seed(chain.cfg, layer, which, KIND_NORM)
    return (0.5 + gen.uniform(seed, 0, n)).astype(np.float32)


def chain_input(chain) -> np.ndarray:
    """The token's hidden state entering layer 0: fp32 N(0, 1) [hidden]."""
    return gen.normal(gen.tensor_seed(chain.cfg, 0, 0, KIND_X), 0, chain.hidden).astype(np.float32)


def dense_weight(cfg: int, layer: int, proj: int, N: int, Kin: int, sigma: float = 0.02) -> np.ndarray:
    """A dense fp32 weight [N][Kin] to ternarize: N(0, sigma^2) (the scale of a
    trained LLM linear's weights; no trained weights exist here)."""
    seed = gen.tensor_seed(cfg, layer, proj, KIND_DENSE)
    return (gen.normal(seed, 0, N * Kin) * sigma).astype(np.float32).reshape(N, Kin)


# Mixture-of-experts decode: routing, expert weights and the tokens' activations.
# A layer's routing gives every token top_k distinct experts, uniformly: the
# experts holding its top_k smallest of one uniform draw per expert (the
# pages give no router; a trained one is skewed, which only moves tokens
# between experts).  Expert e's inputs are the rows of its tokens, in token
# order: the hidden states for gate and up, and for down one row per
# (token, expert) pair of the intermediate activations.
MOE_HIDDEN_ID, MOE_INTER_ID = 0xFFFF, 0xFFFE


def moe_routing(moe, layer: int) -> np.ndarray:
    """int64 [batch][top_k]: each token's experts, ascending."""
    seed = gen.tensor_seed(moe.cfg, layer, 0, KIND_ROUTE)
    E = moe.experts
    out = np.empty((moe.batch, moe.top_k), dtype=np.int64)
    for t in range(moe.batch):
        keys = gen.uniform(seed, t * E, E)
        out[t] = np.sort(np.argsort(keys, kind="stable")[:moe.top_k])
    return out


def moe_expert_rows(moe, layer: int):
    """Per expert: (tokens, pairs), int64 arrays of the batch rows of its
    tokens and of their rows in the intermediate activations (token * top_k
    + the expert's place among the token's experts)."""
    route = moe_routing(moe, layer)
    toks = [[] for _ in range(moe.experts)]
    pairs = [[] for _ in range(moe.experts)]
    for t in range(moe.batch):
        for j, e in enumerate(route[t]):
            toks[int(e)].append(t)
            pairs[int(e)].append(t * moe.top_k + j)
    return [(np.array(a, dtype=np.int64), np.array(b, dtype=np.int64)) for a, b in zip(toks, pairs)]


def moe_hidden(moe, layer: int) -> np.ndarray:
    """The batch's hidden states entering a layer's experts [batch][hidden]
    (fp32 values or bf16 bits, as ``activations``)."""
    return activations(gen.tensor_seed(moe.cfg, layer, MOE_HIDDEN_ID, KIND_X), moe.batch, moe.hidden,
                       F32 if moe.x_type in (F32, I8) else BF16)


def moe_inter(moe, layer: int) -> np.ndarray:
    """The intermediate activations entering the down matrices, one row per
    (token, expert) pair [batch * top_k][inter]."""
    return activations(gen.tensor_seed(moe.cfg, layer, MOE_INTER_ID, KIND_X), moe.batch * moe.top_k,
                       moe.inter, F32 if moe.x_type in (F32, I8) else BF16)


def moe_projection(moe, layer: int, expert: int, proj: int, rows=None) -> dict:
    """Weights of projection ``proj`` (0 gate, 1 up, 2 down) of one expert, as
    ``projection`` draws them (no x)."""
    _, N, Kin = moe.proj_shapes()[proj]
    return projection(moe.case(), layer, expert * 3 + proj, N, Kin, rows=rows, M=0)


__all__ = ["moe_routing", "moe_expert_rows", "moe_hidden", "moe_inter", "moe_projection",
           "projection", "dense_weight", "chain_projection", "chain_norm", "chain_input", "activations", "plane_values", "plane_values_full", "group_scales",
           "tensor_scales", "codebook_indices", "seeds", "N_CODEBOOK",
           "TENSOR", "GROUP_F16", "CODEBOOK", "F32", "BF16", "I8"]
