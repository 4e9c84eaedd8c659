"""The workloads: projection shapes of the two model stacks and the five cases.

Shapes:
  BitNet b1.58-2B-4T (QORA-LLM-2B page, "Architecture" table): hidden 2560,
  30 layers, 20 query / 5 KV heads of 128, FFN 6912.  The seven ternary
  linears of a layer (the "SubLN Pattern" listing on the same page) are
  q, k, v, o, gate, up, down.
  Llama-3.1-8B (the balanced-ternary model card names the model; its
  dimensions are the published ones): hidden 4096, 32 layers, 32 query /
  8 KV heads of 128, FFN 14336.

  Qwen3-30B-A3B (the sasori page's "Measured results" runs it as TQ3P, K=3,
  g=256; the page gives no dimensions, these are the published ones): 48
  layers, hidden 2048, 128 experts of intermediate 768, 8 routed per token.

Each projection is (name, out_features N, in_features Kin), weight N x Kin.
"""
from __future__ import annotations

from dataclasses import dataclass, field

BITNET_2B = {
    "layers": 30,
    "proj": [
        ("q", 2560, 2560),
        ("k", 640, 2560),
        ("v", 640, 2560),
        ("o", 2560, 2560),
        ("gate", 6912, 2560),
        ("up", 6912, 2560),
        ("down", 2560, 6912),
    ],
}

LLAMA_8B = {
    "layers": 32,
    "proj": [
        ("q", 4096, 4096),
        ("k", 1024, 4096),
        ("v", 1024, 4096),
        ("o", 4096, 4096),
        ("gate", 14336, 4096),
        ("up", 14336, 4096),
        ("down", 4096, 14336),
    ],
}

# Scale layouts and activation types, mirroring the C ABI enums.
TENSOR, GROUP_F16, CODEBOOK = 0, 1, 2
F32, BF16, I8 = 0, 1, 2

# Tensor kinds (low 16 bits of the seed key).
KIND_TRITS, KIND_SCALES, KIND_X, KIND_INDEX, KIND_DIGITS, KIND_NORM, KIND_DENSE, KIND_ROUTE = 1, 2, 3, 4, 5, 6, 7, 8


@dataclass(frozen=True)
class Case:
    cfg: int                 # 1..5 (5 = prefill int8, 6 = prefill bf16)
    name: str
    model: dict | None       # stack, or None for the single tiny linear
    planes: int
    group: int               # 0 for per-tensor
    layout: int
    x_type: int
    M: int
    single: tuple = field(default=None)   # (N, Kin) when model is None

    def projections(self):
        """[(layer, proj_index, name, N, Kin)] in stack order."""
        if self.model is None:
            return [(0, 0, "linear", self.single[0], self.single[1])]
        out = []
        for layer in range(self.model["layers"]):
            for p, (nm, n, kin) in enumerate(self.model["proj"]):
                out.append((layer, p, nm, n, kin))
        return out


CASES = {
    "cfg1": Case(1, "tiny single ternary linear 256x512, K=1, g=64, f16 group scales, fp32 x",
                 None, 1, 64, GROUP_F16, F32, 1, single=(256, 512)),
    "cfg2": Case(2, "BitNet b1.58-2B decode stack, 30 layers x 7 projections, K=1, per-tensor scale, int8 x",
                 BITNET_2B, 1, 0, TENSOR, I8, 1),
    "cfg3": Case(3, "Llama-3.1-8B-shaped decode stack, 32 layers x 7 projections, K=3, g=256, f16 group scales, bf16 x",
                 LLAMA_8B, 3, 256, GROUP_F16, BF16, 1),
    "cfg4": Case(4, "balanced-ternary d=3 codec on Llama-3.1-8B shapes, g=16, 27-entry f16 codebook, bf16 x",
                 LLAMA_8B, 3, 16, CODEBOOK, BF16, 1),
    "cfg5a": Case(5, "BitNet b1.58-2B prefill stack, M=2048, K=1, per-tensor scale, int8 x",
                  BITNET_2B, 1, 0, TENSOR, I8, 2048),
    "cfg5b": Case(6, "Llama-3.1-8B-shaped prefill stack, M=512, K=3, g=256, f16 group scales, bf16 x",
                  LLAMA_8B, 3, 256, GROUP_F16, BF16, 512),
}


@dataclass(frozen=True)
class Chain:
    """BitNet b1.58 layers run back to back as one decode chain for one token.

    The layer is the QORA-LLM-2B page's "SubLN Pattern" listing: input
    RMSNorm, q/k/v, attention, attention-sub RMSNorm, o, residual;
    post-attention RMSNorm, gate/up, squared ReLU, FFN-sub RMSNorm, down,
    residual.  The projections' weights follow the BitNet decode stack's
    recipe (one plane, per-tensor scale) and, with ``weights_cfg`` = 2 and the
    BitNet shapes, are the very tensors of that stack.
    """
    cfg: int
    name: str
    layers: int
    hidden: int
    inter: int
    n_heads: int
    n_kv: int
    head_dim: int
    weights_cfg: int
    eps: float = 1e-5

    def proj_shapes(self):
        """[(name, N, Kin)] in the order q, k, v, o, gate, up, down."""
        nq, nkv = self.n_heads * self.head_dim, self.n_kv * self.head_dim
        return [("q", nq, self.hidden), ("k", nkv, self.hidden), ("v", nkv, self.hidden),
                ("o", self.hidden, nq), ("gate", self.inter, self.hidden), ("up", self.inter, self.hidden),
                ("down", self.hidden, self.inter)]

    def dims(self):
        return (self.hidden, self.inter, self.n_heads, self.n_kv, self.head_dim, self.eps)

    def norm_sizes(self):
        """Lengths of the four RMSNorm weights: input, attention-sub, post-attention, FFN-sub."""
        return (self.hidden, self.n_heads * self.head_dim, self.hidden, self.inter)


CHAINS = {
    "chain": Chain(7, "BitNet b1.58-2B decode chain, 30 layers, one token at position 0",
                   30, 2560, 6912, 20, 5, 128, weights_cfg=2),
    "chain_small": Chain(8, "BitNet-shaped decode chain at small sizes, 6 layers",
                         6, 256, 704, 4, 2, 64, weights_cfg=8),
    # widths that are not multiples of the 64-row block (240, 48 and 720):
    # the last block of every projection is partly padding
    "chain_ragged": Chain(9, "decode chain with ragged widths, 3 layers",
                          3, 240, 720, 5, 1, 48, weights_cfg=9),
}


@dataclass(frozen=True)
class Moe:
    """The routed experts of mixture-of-experts layers, decoded for a batch of
    tokens.  Each expert has its own gate, up and down matrices, each fit on
    its own into K planes (sasori page, "How it works & paper"); a token is
    sent to ``top_k`` of the ``experts`` experts of every layer."""
    cfg: int
    name: str
    layers: int
    hidden: int
    inter: int
    experts: int
    top_k: int
    planes: int
    group: int
    layout: int
    x_type: int
    batch: int               # tokens decoded together

    def proj_shapes(self):
        """[(name, N, Kin)] of one expert: gate, up, down."""
        return [("gate", self.inter, self.hidden), ("up", self.inter, self.hidden),
                ("down", self.hidden, self.inter)]

    def case(self) -> Case:
        """The weight recipe of the decode stacks, for the generators."""
        return Case(self.cfg, self.name, None, self.planes, self.group, self.layout, self.x_type, 0,
                    single=(self.hidden, self.hidden))


MOES = {
    "moe": Moe(9, "Qwen3-30B-A3B-shaped MoE experts, 48 layers x 128 experts (8 routed per token), "
                  "K=3, g=256, f16 group scales, int8 x (per-token absmax)", 48, 2048, 768, 128, 8, 3, 256,
               GROUP_F16, I8, 64),
    "moe_small": Moe(10, "MoE experts at small sizes, 2 layers x 16 experts (4 routed per token)",
                     2, 512, 256, 16, 4, 3, 128, GROUP_F16, BF16, 12),
}
