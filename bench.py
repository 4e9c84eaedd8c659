"""Benchmark of the packed ternary-weight decode path on one MI355X.

A step is one pass of the hot path over a whole layer stack for one token:
per-token int8 quantisation of every projection's input (tq_act_quant_int8)
and the ternary GEMV of all projections in one grouped launch
(tq_gemv_grouped_run).  The default workload is the BitNet b1.58-2B decode
stack (30 layers x q,k,v,o,gate,up,down; one trit plane, per-tensor scale,
int8 activations, int32 accumulate), inputs seeded and synthetic, resident in
HBM before timing starts.

Prints one JSON line.  `value` is effective HBM bandwidth: the algorithmic
bytes of a step (packed trits, scales, activations in and out) divided by the
step time.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from synth import device, gen, inputs  # noqa: E402
from synth.configs import BF16, CASES, CHAINS, CODEBOOK, F32, GROUP_F16, I8, TENSOR  # noqa: E402

CODEBOOK_B3 = 3   # the codec with compact base-3 codes (tq.h)

HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "ternary_weight_amd", "csrc")
METRIC = "ternary GEMV effective HBM GB/s (% of peak) at BitNet-2B/Llama-8B shapes, M=1"
METRIC_PREFILL = "ternary prefill GEMM effective TOP/s (MFMA utilisation) at BitNet-2B/Llama-8B shapes"
METRIC_MOE = "MoE expert-grouped ternary GEMV effective HBM GB/s (% of peak), Qwen3-30B-A3B expert shapes"
METRIC_CHAIN = "BitNet-2B decode chain effective HBM GB/s (% of peak), one token through every layer"
MFMA_PEAK_I8_TOPS = 5000.0      # dense int8 MFMA, MI355X
MFMA_PEAK_BF16_TFLOPS = 2500.0  # dense bf16 MFMA, MI355X


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--spin-up-ms", type=float, default=150.0,
                    help="plain streaming reads before the warmup steps: the GPU needs ~20 ms of "
                         "memory load to leave its idle clocks")
    ap.add_argument("--config", default="cfg2", choices=["cfg2", "cfg3", "cfg4", "cfg5a", "cfg5b", "chain",
                                                         "moe", "ternarize", "ternarize_codec"],
                    help="cfg2-4: decode stacks (tq_gemv_grouped_*); cfg5a/b: prefill stacks (tq_gemm_grouped_*); "
                         "chain: the BitNet b1.58-2B layers as a dependent decode chain (tq_bitnet_chain_*)")
    ap.add_argument("--workgroups", type=int, default=0, help="chain: grid of the persistent launch (0 = default)")
    ap.add_argument("--batch", type=int, default=0, help="moe: tokens decoded together (0 = 64)")
    ap.add_argument("--moe-x", choices=["i8", "bf16", "f32"], default="i8",
                    help="moe: activations (i8: fp32 rows quantised per token by the quantiser, or inside "
                         "the product with --fused)")
    ap.add_argument("--M", type=int, default=1, help="decode stacks (cfg2-4): tokens per step, 1 to 16 (more: "
                                                     "the prefill kernels)")
    ap.add_argument("--b3", action="store_true",
                    help="cfg4: pack the codec with compact base-3 codes (TQ_SCALE_CODEBOOK_B3) instead of two-bit "
                         "digit planes")
    ap.add_argument("--waves", type=int, default=0, help="waves per 64-row block in the grouped launch")
    ap.add_argument("--row-blocks", type=int, default=0, help="64-row blocks per workgroup")
    ap.add_argument("--fused", action="store_true",
                    help="int8 path as one call: fp32 activations quantised inside the grouped product "
                         "(TQ_F32_Q8); default is two launches, the batched quantiser then the product")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-legs", action="store_true",
                    help="cfg2 at one token: leave out the Llama-8B-shaped one-token stacks (cfg3, cfg4) that the "
                         "line otherwise carries under 'legs'")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="seconds of oracle work per CPU baseline (a bounded sample of the workload)")
    ap.add_argument("--secondary", action="store_true",
                    help="decode and prefill stacks: add secondary timings after the timed region (single passes "
                         "of the product, cold after a 1 GiB evicting read and warm, the quantiser alone, the "
                         "projections as single launches in a HIP graph, the one-thread oracle)")
    ap.add_argument("--ceiling", action="store_true",
                    help="also time a plain HBM read (torch sum) and copy of 2 GiB as a practical ceiling")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# Workload construction (all on the GPU).
# ---------------------------------------------------------------------------
class Stack:
    """Every projection of a case packed in one slab, with its activations and outputs."""

    def __init__(self, case, M: int, fused: bool = True, b3: bool = False):
        import torch
        from ternary_weight_amd import tq
        self.case, self.M = case, M
        # the codec's weights packed with compact base-3 codes (same canonical arrays)
        self.b3 = b3 and case.layout == CODEBOOK
        self.pack_layout = CODEBOOK_B3 if self.b3 else case.layout
        self.prefill = M > 16          # matrix-core product (tq_gemm) instead of the decode kernels
        # int8 activations: quantise inside the product (one launch per step) or as a separate call
        self.fused = fused and case.x_type == I8 and not self.prefill
        self.run_type = tq.F32_Q8 if self.fused else case.x_type
        self.projs = case.projections()
        K, g, layout = case.planes, case.group, self.pack_layout
        ncb = inputs.N_CODEBOOK if case.layout == CODEBOOK else 0
        self.descs = [tq.desc(K, g, layout, n, kin, n_codebook=ncb) for (_, _, _, n, kin) in self.projs]
        sizes = [tq.packed_size(d) for d in self.descs]
        offs = np.concatenate([[0], np.cumsum([(s + 255) // 256 * 256 for s in sizes])])
        self.slab = torch.empty(int(offs[-1]), dtype=torch.uint8, device="cuda")
        self.blobs = [self.slab[int(offs[i]):int(offs[i]) + sizes[i]] for i in range(len(sizes))]
        self.blob_bytes = int(offs[-1])
        # activations grouped by in_features so that quantisation is one launch per width
        self.widths = sorted({kin for (_, _, _, _, kin) in self.projs})
        self.rows_of = {w: [i for i, p in enumerate(self.projs) if p[4] == w] for w in self.widths}
        act_fp = torch.float32 if case.x_type in (F32, I8) else torch.int16
        self.x_raw = {w: torch.empty((len(self.rows_of[w]) * M, w), dtype=act_fp, device="cuda")
                      for w in self.widths}
        unfused_i8 = case.x_type == I8 and not self.fused
        self.x_q = {w: torch.empty((len(self.rows_of[w]) * M, w), dtype=torch.int8, device="cuda")
                    for w in self.widths} if unfused_i8 else None
        self.x_s = {w: torch.empty(len(self.rows_of[w]) * M, dtype=torch.float32, device="cuda")
                    for w in self.widths} if unfused_i8 else None
        self.ys = [torch.empty((M, n), dtype=torch.float32, device="cuda") for (_, _, _, n, _) in self.projs]
        self.slot = {}
        for w in self.widths:
            for j, i in enumerate(self.rows_of[w]):
                self.slot[i] = (w, j)
        for i, (layer, p, _, n, kin) in enumerate(self.projs):
            d = device.projection(case, layer, p, n, kin, M=M)
            tq.pack(self.descs[i], d["trits"], d["scales"], d["codebook"], self.blobs[i])
            w, j = self.slot[i]
            self.x_raw[w][j * M:(j + 1) * M].copy_(d["x"])
            del d
        torch.cuda.synchronize()
        # grouped plan over the whole stack
        items = []
        for i in range(len(self.projs)):
            w, j = self.slot[i]
            if self.x_q is not None:
                x, xs = self.x_q[w][j * M:(j + 1) * M], self.x_s[w][j * M:(j + 1) * M]
            else:
                x, xs = self.x_raw[w][j * M:(j + 1) * M], None
            items.append((self.descs[i], self.blobs[i], x, xs, self.ys[i], None))
        self._probs = tq.problems(items)
        nbytes = (tq.gemm_grouped_workspace_size(self._probs, M, self.run_type) if self.prefill
                  else tq.gemv_grouped_workspace_size(self._probs, M))
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        self.plan = None
        self._segments = None

    def prepare(self, waves: int = 0, row_blocks: int = 0):
        from ternary_weight_amd import tq
        if self.prefill:
            self.plan = tq.gemm_grouped_prepare(self._probs, self.M, self.run_type, self.ws, self.ws.numel())
            return
        self.plan = tq.gemv_grouped_prepare(self._probs, self.M, self.run_type, self.ws,
                                            self.ws.numel(), waves=waves, row_blocks=row_blocks)

    def quantize(self):
        from ternary_weight_amd import tq
        if self.x_q is None:
            return
        if self._segments is None:
            self._segments = [(self.x_raw[w].shape[0], w, F32, self.x_raw[w], self.x_q[w], self.x_s[w])
                              for w in self.widths]
        tq.act_quant_int8_batch(self._segments)

    def gemv(self):
        from ternary_weight_amd import tq
        (tq.gemm_grouped_run if self.prefill else tq.gemv_grouped_run)(self.plan)

    def ops(self) -> int:
        """Algorithmic operations of the product: 2 M N Kin per plane (multiply-add counted as two)."""
        return sum(2 * self.M * n * kin * self.case.planes for (_, _, _, n, kin) in self.projs)

    # algorithmic bytes ------------------------------------------------------
    def gemv_bytes(self) -> int:
        K, g, layout, M = self.case.planes, self.case.group, self.case.layout, self.M
        # activations as the product reads them: fp32 when it quantises them itself
        xsz = 4 if self.fused else {I8: 1, BF16: 2, F32: 4}[self.case.x_type]
        total = 0
        for (_, _, _, n, kin) in self.projs:
            # packed trits, 2 bits each; compact base-3 codec: 10 bits per two weights
            b = 5 * n * kin // 8 if self.b3 else K * n * kin // 4
            if layout == TENSOR:
                b += 4 * K
            elif layout == GROUP_F16:
                b += 2 * K * n * (kin // g)                    # one f16 per plane, row, group
            else:
                b += (5 * n * (kin // g) + 7) // 8 + 2 * inputs.N_CODEBOOK   # 5-bit index per group
            b += M * kin * xsz + (4 * M if (self.case.x_type == I8 and not self.fused) else 0)
            b += 4 * M * n                                     # fp32 y
            total += b
        return total

    def quant_bytes(self) -> int:
        if self.x_q is None:
            return 0
        return sum(self.M * kin * (4 + 1) + 4 * self.M for (_, _, _, _, kin) in self.projs)


class MoeStack:
    """The routed experts of every MoE layer for one decode batch.

    Every expert's gate, up and down matrices are packed on their own (all
    experts of all layers stay resident, as in a served model); the batch's
    tokens are gathered per expert, in expert order, into one buffer per
    layer and input width; one grouped launch (tq_gemv_grouped_prepare_tokens)
    computes every (layer, expert, projection) that has tokens, each with its
    own token count.  An expert with more than 16 tokens is split into
    problems of at most 16 that share its blob.  int8 activations are
    quantised per token by one tq_act_quant_int8_batch launch over every
    layer's gathered rows (two segments: hidden and intermediate width)
    before the product, or, with ``fused``, inside it (TQ_F32_Q8)."""

    MAX_TOKENS = 16

    def __init__(self, moe, fused: bool = False):
        import torch
        from ternary_weight_amd import tq
        self.moe = moe
        K, g, layout = moe.planes, moe.group, moe.layout
        self.shapes = moe.proj_shapes()
        self.descs = [tq.desc(K, g, layout, n, kin) for (_, n, kin) in self.shapes]
        sizes = [tq.packed_size(d) for d in self.descs]
        self.sizes = sizes
        aligned = [(s + 255) // 256 * 256 for s in sizes]
        self.expert_bytes = sum(aligned)
        self.proj_off = [0, aligned[0], aligned[0] + aligned[1]]
        E, L = moe.experts, moe.layers
        self.slab = torch.empty(L * E * self.expert_bytes, dtype=torch.uint8, device="cuda")
        self.blob_bytes = self.slab.numel()
        for layer in range(L):
            for e in range(E):
                for p in range(3):
                    d = device.moe_projection(moe, layer, e, p)
                    tq.pack(self.descs[p], d["trits"], d["scales"], None, self.blob(layer, e, p))
                    del d
        torch.cuda.synchronize()
        self.fused = fused and moe.x_type == I8
        self.run_type = {BF16: BF16, F32: F32, I8: tq.F32_Q8 if self.fused else I8}[moe.x_type]
        self.routes = [inputs.moe_expert_rows(moe, layer) for layer in range(L)]
        rows = moe.batch * moe.top_k
        # every layer's gathered rows in one matrix per width: [layers * rows][width]
        xh = [device.moe_hidden(moe, layer).index_select(0, torch.from_numpy(
              np.concatenate([a for a, _ in self.routes[layer]])).cuda()) for layer in range(L)]
        xi = [device.moe_inter(moe, layer).index_select(0, torch.from_numpy(
              np.concatenate([b for _, b in self.routes[layer]])).cuda()) for layer in range(L)]
        self.xh_all, self.xi_all = torch.cat(xh).contiguous(), torch.cat(xi).contiguous()
        del xh, xi
        self.quant = moe.x_type == I8 and not self.fused
        if self.quant:
            self.qh = torch.empty(self.xh_all.shape, dtype=torch.int8, device="cuda")
            self.qi = torch.empty(self.xi_all.shape, dtype=torch.int8, device="cuda")
            self.sh = torch.empty(self.xh_all.shape[0], dtype=torch.float32, device="cuda")
            self.si = torch.empty(self.xi_all.shape[0], dtype=torch.float32, device="cuda")
            self._segments = [(self.xh_all.shape[0], moe.hidden, F32, self.xh_all, self.qh, self.sh),
                              (self.xi_all.shape[0], moe.inter, F32, self.xi_all, self.qi, self.si)]
        self.ys = []
        items, tokens, self.meta = [], [], []
        for layer in range(L):
            r = self.routes[layer]
            self.ys.append([torch.empty((rows, n), dtype=torch.float32, device="cuda") for (_, n, _) in self.shapes])
            off = 0
            for e in range(E):
                n_e = len(r[e][0])
                for c in range(0, n_e, self.MAX_TOKENS):
                    m = min(self.MAX_TOKENS, n_e - c)
                    a = off + c
                    g0 = layer * rows + a          # first row in the all-layer matrices
                    for p in range(3):
                        if self.quant:
                            x = (self.qh if p < 2 else self.qi)[g0:g0 + m]
                            xs = (self.sh if p < 2 else self.si)[g0:g0 + m]
                        else:
                            x, xs = (self.xh_all if p < 2 else self.xi_all)[g0:g0 + m], None
                        items.append((self.descs[p], self.blob(layer, e, p), x, xs, self.ys[layer][p][a:a + m], None))
                        tokens.append(m)
                        self.meta.append((layer, e, p, a, m))
                off += n_e
        torch.cuda.synchronize()
        self.tokens = tokens
        self.max_tokens = max(tokens) if tokens else 0
        self._probs = tq.problems(items)
        nbytes = tq.gemv_grouped_workspace_size(self._probs, self.max_tokens)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        self.plan = None

    def blob(self, layer, e, p):
        o = (layer * self.moe.experts + e) * self.expert_bytes + self.proj_off[p]
        return self.slab[o:o + self.sizes[p]]

    def prepare(self, waves: int = 0, row_blocks: int = 0):
        from ternary_weight_amd import tq
        self.plan = tq.gemv_grouped_prepare_tokens(self._probs, self.tokens, self.run_type, self.ws,
                                                   self.ws.numel(), waves=waves, row_blocks=row_blocks)

    def quantize(self):
        from ternary_weight_amd import tq
        if self.quant:
            tq.act_quant_int8_batch(self._segments)

    def gemv(self):
        from ternary_weight_amd import tq
        tq.gemv_grouped_run(self.plan)

    def active_experts(self) -> int:
        return sum(sum(1 for a, _ in r if len(a)) for r in self.routes)

    def gemv_bytes(self) -> int:
        """Algorithmic bytes of a step: the packed trits and scales of every
        routed expert once, each routed token's input rows once (the hidden
        state read by gate and up counts once) and every output written."""
        moe, K = self.moe, self.moe.planes
        xsz = {BF16: 2, F32: 4, I8: 4}[moe.x_type]
        w = 0
        for (_, n, kin) in self.shapes:
            w += K * n * kin // 4
            w += 2 * K * n * (kin // moe.group) if moe.layout == GROUP_F16 else 4 * K
        pairs = moe.layers * moe.batch * moe.top_k
        if self.quant:
            xsz = 1
        return (self.active_experts() * w + pairs * (moe.hidden + moe.inter) * xsz
                + (pairs * 8 if self.quant else 0) + pairs * 4 * (2 * moe.inter + moe.hidden))

    def quant_bytes(self) -> int:
        """The quantiser's bytes: fp32 rows in, int8 rows and a scale per row out."""
        if not self.quant:
            return 0
        pairs = self.moe.layers * self.moe.batch * self.moe.top_k
        return pairs * (self.moe.hidden + self.moe.inter) * 5 + 8 * pairs


def decode_kernel_name(plan, run_type, layout, planes, group) -> str:
    """The kernel a grouped decode plan launches (as rocprofv3 names it)."""
    if layout == CODEBOOK_B3:
        planes = 1              # the compact codec's kernels take one combined value per weight
    if plan.family >= 1000:     # several tokens: the matrix-core decode kernel
        if run_type == I8:
            ks = 64
        else:
            ks = 32 if layout in (TENSOR, GROUP_F16) and (layout == TENSOR or group % 32 == 0) else 16
        # int8 with one plane and a per-tensor scale from 8 tokens: the wide
        # kernel (two 64-row blocks per wave)
        wide = run_type == I8 and layout == TENSOR and planes == 1 and plan.M >= 8
        return "k_gemm_skinny%s_grouped<%d, %d, %d, %d>" % ("_wide" if wide else "", run_type, layout, planes, ks)
    mt = 1 if plan.M <= 1 else 4
    kind = "k_gemv_wave_items" if plan.mode == 1 else "k_gemv_grouped"   # an item per wave, or per workgroup
    return "%s<%d, %d, %d, %d>" % (kind, run_type, layout, planes, mt)


# ---------------------------------------------------------------------------
# Parity spot check and CPU baseline (oracle).
# ---------------------------------------------------------------------------
def rel_err(y, ystar) -> float:
    """max over tokens of max_n |y - y*| / max(|y*|, rms(y*))."""
    y, ystar = np.asarray(y, np.float64), np.asarray(ystar, np.float64)
    worst = 0.0
    for m in range(ystar.shape[0]):
        den = np.maximum(np.abs(ystar[m]), np.sqrt(np.mean(ystar[m] ** 2)))
        den = np.where(den == 0, 1.0, den)
        worst = max(worst, float(np.max(np.abs(y[m] - ystar[m]) / den)))
    return worst


def spot_check(stack, n_proj=3, rows=64) -> dict:
    """Rows of a few projections against the oracle on host-regenerated inputs."""
    import oracle
    import torch
    case, M = stack.case, stack.M
    rng = np.random.default_rng(99)
    picks = sorted({0, len(stack.projs) - 1, int(rng.integers(len(stack.projs)))})[:n_proj]
    worst, exact = 0.0, True
    for i in picks:
        layer, p, _, n, kin = stack.projs[i]
        r = np.sort(rng.choice(n, size=min(rows, n), replace=False))
        h = inputs.projection(case, layer, p, n, kin, rows=r, M=M)
        y = stack.ys[i].detach().cpu().numpy()[:, r]
        if case.x_type == I8:
            q, s = oracle.act_quant_i8(h["x"], F32)
            out = oracle.gemv_i8(case.planes, case.group, case.layout, h["trits"], h["scales"], q, s,
                                 h["codebook"])
            exact &= bool(np.array_equal(y.view(np.uint32), out["y32"].view(np.uint32)))
        else:
            ref = oracle.gemv_fp(case.planes, case.group, case.layout, h["trits"], h["scales"], h["x"],
                                 BF16 if case.x_type == BF16 else F32, h["codebook"])
            worst = max(worst, rel_err(y, ref))
    torch.cuda.synchronize()
    return {"projections": len(picks), "rows_each": rows,
            "bit_exact" if case.x_type == I8 else "max_rel_err": exact if case.x_type == I8 else worst}


def oracle_threads() -> int:
    """Host threads for the oracle baseline: the process's CPU share as the
    job sets it (OMP_NUM_THREADS), else every core the process may run on."""
    try:
        n = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        n = 0
    return n if n > 0 else len(os.sched_getaffinity(0))


def cpu_baseline_prefill(stack, seconds: float, tokens: int = 32) -> dict:
    """The oracle on the host cores: the first projection of the stack for its first `tokens` tokens,
    repeated for about `seconds`, as operations per second."""
    import oracle
    case = stack.case
    threads = oracle_threads()
    orc = oracle.default()
    layer, p, name, n, kin = stack.projs[0]
    h = inputs.projection(case, layer, p, n, kin, M=tokens)
    K, g, layout = case.planes, case.group, case.layout
    ops, reps, t0 = 0, 0, time.perf_counter()
    while True:
        if case.x_type == I8:
            q, s = orc.act_quant_i8(h["x"], F32)
            orc.gemv_i8(K, g, layout, h["trits"], h["scales"], q, s, h["codebook"], nthreads=threads)
        else:
            orc.gemv_fp(K, g, layout, h["trits"], h["scales"], h["x"], case.x_type, h["codebook"], nthreads=threads)
        ops += 2 * tokens * n * kin * K
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(ops / el / 1e12, 6), "unit": "TOP/s" if case.x_type == I8 else "TFLOP/s",
            "cores": threads, "kind": "oracle",
            "sample": "projection %s of layer 0 (%d x %d, %d plane(s)) for the first %d tokens, %d repetitions, "
                      "%.1f s; C oracle, OpenMP over output rows" % (name, n, kin, K, tokens, reps, el)}


def canonical_inputs(case, layer, p, n, kin, M) -> dict:
    """Host copies of the canonical arrays of one projection, drawn by the
    device copy of the seeded generator (bit-identical to the host one, which
    is too slow for whole layers of the 8B-shaped stacks)."""
    d = device.projection(case, layer, p, n, kin, M=M)
    h = {"trits": d["trits"].cpu().numpy()}
    sc = d["scales"].cpu().numpy()
    h["scales"] = sc.view(np.uint16) if case.layout == GROUP_F16 else sc
    h["codebook"] = None if d["codebook"] is None else d["codebook"].cpu().numpy().view(np.uint16)
    x = d["x"].cpu().numpy()
    h["x"] = x.view(np.uint16) if case.x_type == BF16 else x
    return h


def cpu_baseline(stack, seconds: float) -> dict:
    """The oracle on the host cores, over whole layers of the same stack."""
    import oracle
    case, M = stack.case, stack.M
    if stack.prefill:
        return cpu_baseline_prefill(stack, seconds)
    threads = oracle_threads()
    orc = oracle.default()
    # layer 0 of the stack, every projection
    per_layer = len(case.model["proj"])
    layer_inputs = []
    for (layer, p, _, n, kin) in stack.projs[:per_layer]:
        layer_inputs.append((n, kin, canonical_inputs(case, layer, p, n, kin, M)))
    done_bytes, t0, reps = 0, time.perf_counter(), 0
    layer_bytes = 0
    K, g, layout = case.planes, case.group, case.layout
    for (n, kin, h) in layer_inputs:
        xsz = {I8: 1, BF16: 2, F32: 4}[case.x_type]
        layer_bytes += K * n * kin // 4 + M * kin * xsz + 4 * M * n + (M * kin * 5 if case.x_type == I8 else 0)
        if layout == GROUP_F16:
            layer_bytes += 2 * K * n * (kin // g)
        elif layout == CODEBOOK:
            layer_bytes += (5 * n * (kin // g) + 7) // 8 + 2 * inputs.N_CODEBOOK
    while True:
        for (n, kin, h) in layer_inputs:
            if case.x_type == I8:
                q, s = orc.act_quant_i8(h["x"], F32)
                orc.gemv_i8(K, g, layout, h["trits"], h["scales"], q, s, h["codebook"], nthreads=threads)
            else:
                orc.gemv_fp(K, g, layout, h["trits"], h["scales"], h["x"], case.x_type, h["codebook"],
                            nthreads=threads)
        done_bytes += layer_bytes
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(done_bytes / el / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "layer 0 of the stack (first %d projections), %d repetitions, %.1f s; C oracle, "
                      "OpenMP over output rows" % (per_layer, reps, el)}


def release_device():
    """Wait for all queued work and return the freed buffers to the device."""
    import gc
    import torch
    torch.cuda.synchronize()
    gc.collect()
    torch.cuda.empty_cache()
    torch.cuda.synchronize()


def spin_up(ms: float, nbytes: int = 1 << 30):
    """Keep HBM busy for about `ms` with the harness read kernel (not timed, not a step)."""
    import torch
    if ms <= 0:
        return
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            device.stream_read(buf, sink, 8192)
        torch.cuda.synchronize()
    del buf


def hbm_ceiling(nbytes: int = 4 << 30, reps: int = 5) -> dict:
    """A plain streaming read (harness kernel) and a device copy (torch) of known size."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = {"bytes": nbytes}
    for blocks in (2048, 8192):
        device.stream_read(a, sink, blocks)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            device.stream_read(a, sink, blocks)
        e1.record()
        torch.cuda.synchronize()
        out["read_GBs_%d" % blocks] = round(nbytes * reps / (e0.elapsed_time(e1) / 1e3) / 1e9, 1)
    half = nbytes // 2
    src, dst = a[:half], a[half:]
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    out["copy_GBs"] = round(2 * half * reps / (e0.elapsed_time(e1) / 1e3) / 1e9, 1)
    del a
    return out


# ---------------------------------------------------------------------------
# rocprofv3 summaries (profiles/) and the measured HBM traffic of the kernel.
# ---------------------------------------------------------------------------
# Sources that make up each kernel family (the traffic of a kernel is reused
# only while none of them has changed).
_COMMON_SOURCES = ["tq_decode.h", "tq_internal.h", "tq_layout.h"]
_FAMILY_SOURCES = {
    "k_gemv": ["tq_gemv_impl.h", "tq_gemv.hip", "tq_entry.hip"],
    "k_gemm": ["tq_gemm_impl.h", "tq_gemm_kernels.h", "tq_gemm_skinny.h", "tq_gemm.hip"],
    "k_bitnet_chain": ["tq_chain.hip", "tq_gemv_impl.h"],
    "k_tern": ["tq_ternarize.hip"],
}


def _code_only(text: bytes) -> bytes:
    """Source text without comments and blank space (edits of comments keep a fingerprint)."""
    import re
    t = text.decode("utf-8", "replace")
    t = re.sub(r"/\*.*?\*/", " ", t, flags=re.S)
    t = re.sub(r"//[^\n]*", " ", t)
    return " ".join(t.split()).encode()


def kernel_fingerprint(kernel: str) -> str:
    """Hash of the code of the kernel's family (and the header of the ABI), comments excluded."""
    fam = next((k for k in _FAMILY_SOURCES if kernel.startswith(k)), None)
    files = _COMMON_SOURCES + (_FAMILY_SOURCES[fam] if fam else [])
    prefix = {"k_gemv": "tq_gemv_", "k_gemm": "tq_gemm_"}.get(fam)
    if prefix:
        files += sorted(os.path.basename(f) for f in glob.glob(os.path.join(CSRC, prefix + "*.hip")))
    h = hashlib.sha256()
    for f in sorted(set(files)):
        h.update(f.encode())
        h.update(_code_only(open(os.path.join(CSRC, f), "rb").read()))
    h.update(_code_only(open(os.path.join(ROOT, "include", "tq.h"), "rb").read()))
    return h.hexdigest()[:16]


def _trace_rows(d):
    f = glob.glob(os.path.join(d, "*_kernel_trace.csv"))
    return list(csv.DictReader(open(f[0]))) if f else []


def _pmc_values(d):
    out = {}
    for f in glob.glob(os.path.join(d, "*_counter_collection.csv")):
        for r in csv.DictReader(open(f)):
            out.setdefault((r["Kernel_Name"], r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    return out


def _pmc_means(d):
    return {k: (sum(v) / len(v), len(v)) for k, v in _pmc_values(d).items()}


def summarize(args) -> None:
    """Write a profiles/*.md summary from rocprofv3 output directories."""
    kern = args.kernel
    lines = ["# %s" % args.title, ""]
    rec = {"kernel": kern, "fingerprint": kernel_fingerprint(kern)}
    if args.trace_dir:
        stats = glob.glob(os.path.join(args.trace_dir, "*_kernel_stats.csv"))
        lines += ["Command: `%s`" % args.trace_cmd, "", "rocprofv3 --kernel-trace --stats, top kernels by total time:", "",
                  "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
        rows = list(csv.DictReader(open(stats[0])))
        ranked = sorted(rows, key=lambda r: -float(r["TotalDurationNs"]))
        shown = ranked[:8] + [r for r in ranked[8:] if kern in r["Name"]]
        for r in shown:
            lines.append("| `%s` | %s | %.2f | %.2f | %.2f |" % (r["Name"][:90], r["Calls"], float(r["AverageNs"]) / 1e3,
                                                               float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
        for r in rows:
            if kern in r["Name"]:
                rec["avg_us"] = round(float(r["AverageNs"]) / 1e3, 3)
                rec["calls"] = int(r["Calls"])
        tr = [r for r in _trace_rows(args.trace_dir) if kern in r["Kernel_Name"]]
        if tr:
            tr.sort(key=lambda r: int(r["Start_Timestamp"]))
            if args.timed_launches:
                sel = tr[args.first_launch:args.first_launch + args.timed_launches]
                what = "launches %d .. %d (the timed region)" % (args.first_launch, args.first_launch + len(sel) - 1)
            else:
                sel, what = tr, "all launches"
            d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in sel]
            rec["timed_avg_us"] = round(sum(d) / len(d), 3)
            lines += ["", "Kernel `%s`: average of all %d launches %.2f us; of %s %.2f us."
                      % (kern, len(tr), rec.get("avg_us", float("nan")), what, rec["timed_avg_us"])]
    if args.fetch_dir and args.write_dir:
        f, w = _pmc_means(args.fetch_dir), _pmc_means(args.write_dir)

        def find(tab, name, counter):
            for (k, c), v in tab.items():
                if name in k and c == counter:
                    return v
            return None
        # calibration: the largest dispatch of the harness read and of torch's
        # fill is the one of known size (the smaller ones warm the GPU up or
        # evict the caches)
        def largest(d, name, counter):
            for (k, c), v in _pmc_values(d).items():
                if name in k and c == counter:
                    return (max(v), len(v))
            return None
        read_kib = largest(args.fetch_dir, "k_stream_read", "FETCH_SIZE")
        fill_kib = largest(args.write_dir, "vectorized_elementwise_kernel<16", "WRITE_SIZE")
        gf, gw = find(f, kern, "FETCH_SIZE"), find(w, kern, "WRITE_SIZE")
        fetch_factor = (args.read_bytes / 1024) / read_kib[0]
        write_factor = (args.fill_bytes / 1024) / fill_kib[0]
        traffic = gf[0] * 1024 * fetch_factor + gw[0] * 1024 * write_factor
        rec.update({"fetch_kib": round(gf[0], 1), "write_kib": round(gw[0], 1), "fetch_factor": round(fetch_factor, 4),
                    "write_factor": round(write_factor, 4), "traffic_bytes": int(round(traffic))})
        lines += ["", "Commands: `%s` (FETCH_SIZE) and the same with `--pmc WRITE_SIZE`." % args.pmc_cmd, "",
                  "Calibration with kernels of known size in the same run: the harness streaming read of %d bytes "
                  "reads FETCH_SIZE %.1f KiB (factor %.4f); torch's fill of %d bytes reads WRITE_SIZE %.1f KiB "
                  "(factor %.4f)." % (args.read_bytes, read_kib[0], fetch_factor, args.fill_bytes, fill_kib[0], write_factor),
                  "", "Kernel `%s` per launch (%d launches): FETCH_SIZE %.1f KiB, WRITE_SIZE %.1f KiB -> HBM traffic "
                  "%.0f bytes." % (kern, gf[1], gf[0], gw[0], traffic)]
    for d in args.counters_dir or []:
        tab = _pmc_means(d)
        rows = sorted((c, v) for (k, c), v in tab.items() if kern in k)
        if rows:
            lines += ["", "Counters per launch of `%s` (mean over %d launches), from `%s`:" % (kern, rows[0][1][1],
                                                                                            args.counters_cmd or d),
                      "", "| counter | value |", "|---|---|"]
            for c, (v, _) in rows:
                lines.append("| %s | %.6g |" % (c, v))
                rec.setdefault("counters", {})[c] = v
    lines += ["", "```json", json.dumps(rec), "```", ""]
    open(args.out, "w").write("\n".join(lines))
    print("wrote", args.out)


def measured_traffic(kernel: str):
    """HBM bytes per launch from a profiles/ summary of the current sources, else None."""
    fp = kernel_fingerprint(kernel)
    for f in sorted(glob.glob(os.path.join(PROFILES, "*.md"))):
        text = open(f).read()
        if "```json" not in text:
            continue
        rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
        if rec.get("kernel") == kernel and rec.get("fingerprint") == fp and "traffic_bytes" in rec:
            return rec["traffic_bytes"]
    return None


# ---------------------------------------------------------------------------
# Secondary timings of a decode stack (reported beside the bench line).
# ---------------------------------------------------------------------------
def single_passes(run, reps: int = 20, evict_bytes: int = 0) -> dict:
    """`run` timed alone (events around it) `reps` times: median, min and max
    in microseconds.  With `evict_bytes`, each pass follows an untimed read
    of that many other bytes (more than the 256 MiB MALL; a read, so that no
    dirty lines are written back during the pass), so that no code comes
    from a cache."""
    import torch
    scratch = torch.ones(max(evict_bytes, 16), dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(reps):
        if evict_bytes:
            device.stream_read(scratch, sink, 8192)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    del scratch
    times.sort()
    return {"median_us": round(times[len(times) // 2], 2), "min_us": round(times[0], 2),
            "max_us": round(times[-1], 2), "reps": reps, "evict_bytes": evict_bytes}


def timed_us(run, reps: int = 50) -> float:
    """Average of `run` back to back between one pair of events (microseconds)."""
    import torch
    stream = torch.cuda.current_stream()
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def graph_of_single_launches(stack, replays: int = 20) -> dict:
    """Every projection of the stack as its own tq_gemv launch, captured in
    one HIP graph and replayed: the per-launch alternative to the grouped
    launch (same inputs and outputs)."""
    import torch
    from ternary_weight_amd import tq
    calls = []
    for i, (layer, p, _, n, kin) in enumerate(stack.projs):
        w, j = stack.slot[i]
        M = stack.M
        if stack.x_q is not None:
            x, xs = stack.x_q[w][j * M:(j + 1) * M], stack.x_s[w][j * M:(j + 1) * M]
        else:
            x, xs = stack.x_raw[w][j * M:(j + 1) * M], None
        calls.append((stack.descs[i], stack.blobs[i], M, stack.run_type, x, xs, stack.ys[i]))

    def run_all():
        for (d, blob, M, xt, x, xs, y) in calls:
            tq.gemv(d, blob, M, xt, x, xs, y)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_all()                                   # warm: the first calls query the device
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_all()
    us = timed_us(g.replay, replays)
    eager = timed_us(run_all, replays)
    return {"launches": len(calls), "graph_replay_us": round(us, 2), "eager_launches_us": round(eager, 2)}


def cpu_one_thread(stack, seconds: float = 2.0) -> dict:
    """The oracle on one host thread over the first projection of the stack."""
    import oracle
    case, M = stack.case, stack.M
    orc = oracle.default()
    layer, p, name, n, kin = stack.projs[0]
    h = inputs.projection(case, layer, p, n, kin, M=M)
    K, g, layout = case.planes, case.group, case.layout
    xsz = {I8: 1, BF16: 2, F32: 4}[case.x_type]
    b = K * n * kin // 4 + M * kin * xsz + 4 * M * n
    done, t0 = 0, time.perf_counter()
    while True:
        if case.x_type == I8:
            q, sx = orc.act_quant_i8(h["x"], F32)
            orc.gemv_i8(K, g, layout, h["trits"], h["scales"], q, sx, h["codebook"], nthreads=1)
        else:
            orc.gemv_fp(K, g, layout, h["trits"], h["scales"], h["x"], case.x_type, h["codebook"], nthreads=1)
        done += b
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(done / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "projection %s of layer 0 (%d x %d), %.1f s" % (name, n, kin, el)}


# ---------------------------------------------------------------------------
def main():
    if len(sys.argv) > 1 and sys.argv[1] == "summarize":
        ap = argparse.ArgumentParser(description="write a profiles/ summary from rocprofv3 output")
        ap.add_argument("summarize")
        ap.add_argument("--kernel", required=True)
        ap.add_argument("--title", required=True)
        ap.add_argument("--out", required=True)
        ap.add_argument("--trace-dir")
        ap.add_argument("--trace-cmd", default="")
        ap.add_argument("--timed-launches", type=int, default=0)
        ap.add_argument("--first-launch", type=int, default=0, help="index of the first timed launch of the kernel")
        ap.add_argument("--fetch-dir")
        ap.add_argument("--write-dir")
        ap.add_argument("--pmc-cmd", default="")
        ap.add_argument("--counters-dir", action="append", help="rocprofv3 --pmc output of other counters")
        ap.add_argument("--counters-cmd", default="")
        ap.add_argument("--read-bytes", type=int, default=4 << 30)
        ap.add_argument("--fill-bytes", type=int, default=4 << 30)
        summarize(ap.parse_args())
        return
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only; the multi-GPU path is not built (--gpus %d refused)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.config == "chain":
        main_chain(args)
        return
    if args.config == "moe":
        main_moe(args)
        return
    if args.config.startswith("ternarize"):
        main_ternarize(args)
        return
    M = args.M if args.config in ("cfg2", "cfg3", "cfg4") else CASES[args.config].M
    out = measure_stack(args, args.config, M, fused=args.fused, waves=args.waves, row_blocks=args.row_blocks,
                        spin_up_ms=args.spin_up_ms, secondary=args.secondary, ceiling=args.ceiling, b3=args.b3)
    if args.config == "cfg2" and M == 1 and not args.no_legs:
        # the metric names both shapes: the Llama-8B-shaped one-token stacks
        # are measured the same way, after the BitNet line's own timed region
        # (and the codec once more with its compact base-3 codes)
        out["legs"] = {}
        for key, name, b3 in (("cfg3", "cfg3", False), ("cfg4", "cfg4", False), ("cfg4_b3", "cfg4", True)):
            # each leg's steps are about 0.9 ms: at least 100 ms of them untimed
            # first, so that its 20 or so timed steps do not meet clocks still
            # coming up (5 warm-up steps: 70.7% for cfg3, 100: 74.6%)
            leg = measure_stack(args, name, 1, fused=False, waves=0, row_blocks=0, spin_up_ms=args.spin_up_ms,
                                secondary=False, ceiling=False, b3=b3, min_warmup_ms=100.0)
            out["legs"][key] = {k: leg[k] for k in ("value", "unit", "ms_per_step", "dtype", "tok_per_s_equiv",
                                                    "gemv_us", "roofline", "cold_pass", "cpu_baseline",
                                                    "parity_spot_check", "steps", "warmup")}
            out["legs"][key]["workload"] = leg["config"]["workload"] + (
                ", compact base-3 codes (5 bits per weight)" if b3 else "")
            out["legs"][key]["M"] = 1
    print(json.dumps(out), flush=True)
    release_device()


def measure_stack(args, config, M, fused, waves, row_blocks, spin_up_ms, secondary, ceiling, b3=False,
                  min_warmup_ms: float = 0.0) -> dict:
    """Build one stack, time args.steps steps after args.warmup (and, with
    min_warmup_ms, as many more untimed steps as make that long), and return
    its bench line."""
    import torch
    case = CASES[config]
    t_build = time.perf_counter()
    stack = Stack(case, M, fused=fused, b3=b3)
    stack.prepare(waves, row_blocks)
    build_s = time.perf_counter() - t_build
    print("built %s: %d projections, %.1f MB packed, plan %d items x %d blocks x %d waves (%.1f s)"
          % (config, len(stack.projs), stack.blob_bytes / 1e6, stack.plan.n_items,
             stack.plan.row_blocks, stack.plan.waves, build_s), file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    spin_up(spin_up_ms)
    t_w = time.perf_counter()
    for _ in range(args.warmup):
        stack.quantize()
        stack.gemv()
    torch.cuda.synchronize()
    warmup = args.warmup
    if min_warmup_ms > 0:
        # the clocks come up under the stack's own load: untimed steps until
        # min_warmup_ms have passed
        while (time.perf_counter() - t_w) * 1e3 < min_warmup_ms:
            for _ in range(8):
                stack.quantize()
                stack.gemv()
            torch.cuda.synchronize()
            warmup += 8

    # timed region: K whole steps, events only at its two ends
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        stack.quantize()
        stack.gemv()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / args.steps
    if stack.x_q is None:
        # one launch per step: the step time is the kernel's launch duration
        gemv_avg = ms_step
    else:
        # the product kernel alone, back to back between one pair of events
        reps = max(args.steps, 20)
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(reps):
            stack.gemv()
        g1.record(stream)
        torch.cuda.synchronize()
        gemv_avg = g0.elapsed_time(g1) / reps

    gbytes, qbytes = stack.gemv_bytes(), stack.quant_bytes()
    if stack.prefill:
        step = 64 if case.x_type == I8 else (32 if case.layout == TENSOR or case.group % 32 == 0 else 16)
        # 16 x 16 tiles per wave: 4 x 8 for int8 with one plane and a per-tensor
        # scale (its int32 sums are the result), 4 x 4 otherwise
        fn = 8 if case.x_type == I8 and case.layout == TENSOR and case.planes == 1 else 4
        kernel_name = ("k_gemm_grouped<%d, %d, %d, 4, 4, %d, 2>" % (stack.run_type, CODEBOOK_B3, 1, 16) if stack.b3 else
                       "k_gemm_grouped<%d, %d, %d, 4, %d, %d, 2>" % (stack.run_type, case.layout, case.planes, fn, step))
        ops = stack.ops()
        value = ops / (ms_step / 1e3) / 1e12
        achieved = ops / (gemv_avg / 1e3) / 1e12
        peak = MFMA_PEAK_I8_TOPS if case.x_type == I8 else MFMA_PEAK_BF16_TFLOPS
        unit = "TOP/s" if case.x_type == I8 else "TFLOP/s"
    else:
        kernel_name = decode_kernel_name(stack.plan, stack.run_type, stack.pack_layout, case.planes, case.group)
        value = (gbytes + qbytes) / (ms_step / 1e3) / 1e9
        achieved = gbytes / (gemv_avg / 1e3) / 1e9
        peak, unit = HBM_PEAK_GBS, "GB/s"

    ceil = hbm_ceiling() if ceiling else None
    check = None if args.no_check else spot_check(stack)
    cpu = None if args.no_cpu_baseline else cpu_baseline(stack, args.cpu_seconds)
    # the product alone, one pass at a time, each after an untimed 1 GiB read
    # of other memory (more than the 256 MiB MALL), so that no code comes from
    # a cache: the cold figure beside the back-to-back one
    cold = single_passes(stack.gemv, evict_bytes=1 << 30)
    cold["frac_of_hbm_peak"] = (None if stack.prefill else
                                round(gbytes / (cold["median_us"] / 1e6) / 1e9 / HBM_PEAK_GBS, 4))
    sec = None
    if secondary:
        warm = single_passes(stack.gemv)
        warm["frac_of_hbm_peak"] = (None if stack.prefill else
                                    round(gbytes / (warm["median_us"] / 1e6) / 1e9 / HBM_PEAK_GBS, 4))
        sec = {"single_pass_product": warm}
        if stack.x_q is not None:
            sec["act_quant_us"] = round(timed_us(stack.quantize), 2)
        if not stack.prefill:
            sec["single_launches"] = graph_of_single_launches(stack)
        if not args.no_cpu_baseline:
            sec["cpu_one_thread"] = cpu_one_thread(stack)

    out = {
        "metric": METRIC_PREFILL if stack.prefill else METRIC,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {I8: "i8", BF16: "bf16", F32: "f32"}[case.x_type],
        "data": "synthetic (seeded SplitMix64; trits P(0)=0.4, x ~ N(0,1))",
        "config": {
            "workload": case.name,
            "layers": case.model["layers"],
            "projections": len(stack.projs),
            "M": M,
            "planes": case.planes,
            "group": case.group,
            "scale_layout": {TENSOR: "tensor", GROUP_F16: "group_f16", CODEBOOK: "codebook",
                             CODEBOOK_B3: "codebook_b3"}[stack.pack_layout],
            "step": ("act-quant of every projection input + one grouped MFMA GEMM launch over the stack"
                     if case.x_type == I8 else "one grouped MFMA GEMM launch over the stack") if stack.prefill else
                    ("one grouped launch over the stack; fp32 inputs quantised per token to int8 "
                     "inside it (bit-identical to the separate quantiser)") if stack.fused else
                    ("act-quant of every projection input + one grouped GEMV launch over the stack"
                     if case.x_type == I8 else "one grouped GEMV launch over the stack"),
            "packed_weight_bytes": stack.blob_bytes,
            "grouped_waves": stack.plan.waves,
            "grouped_row_blocks": stack.plan.row_blocks,
        },
        "tok_per_s_equiv": round(M * 1e3 / ms_step, 1),
        "gemv_us": round(gemv_avg * 1e3, 2),
        "roofline": {
            "bound": "mfma" if stack.prefill else "hbm",
            "achieved": round(achieved, 1),
            "peak": peak,
            "unit": unit,
            "frac": round(achieved / peak, 4),
            "traffic": measured_traffic(kernel_name),
            "kernel": kernel_name,
            "bytes_per_launch": gbytes,
            **({"ops_per_launch": stack.ops(),
                "effective_hbm_GBs": round(gbytes / (gemv_avg / 1e3) / 1e9, 1)} if stack.prefill else {}),
        },
        "cpu_baseline": cpu,
        "hbm_ceiling": ceil,
        "parity_spot_check": check,
        "cold_pass": cold,
        "secondary": sec,
        "wall_s_timed": round(wall, 3),
    }
    out["warmup"] = warmup
    del stack
    release_device()
    return out
    print(json.dumps(out), flush=True)
    release_device()


# ---------------------------------------------------------------------------
# The decode chain: one token through every BitNet layer, dependencies kept.
# ---------------------------------------------------------------------------
def chain_bytes(chain, blob_bytes: int) -> int:
    """Algorithmic bytes of one token through the chain: the packed trits and
    scales of every projection, the RMSNorm weights, and each phase's input
    read and output written once (fp32)."""
    sizes = chain.norm_sizes()
    per_layer = 4 * sum(sizes)                                       # norm weights
    nqkv = (chain.n_heads + 2 * chain.n_kv) * chain.head_dim
    per_layer += 4 * (chain.hidden + nqkv)                           # QKV: x in, q|k|v out
    per_layer += 4 * (chain.n_kv * chain.head_dim + 2 * chain.hidden)   # O: v in, x in, x1 out
    per_layer += 4 * (chain.hidden + chain.inter)                    # GU: x1 in, act out
    per_layer += 4 * (chain.inter + 2 * chain.hidden)                # DOWN: act in, x1 in, x out
    trits = sum(n * kin // 4 + 4 for (_, n, kin) in chain.proj_shapes()) * chain.layers
    return trits + per_layer * chain.layers


def chain_spot_check(chain, blobs, norms_dev, dims) -> dict:
    """The first layer on its own plan, against the oracle on host-regenerated inputs."""
    import oracle
    import torch
    from ternary_weight_amd import tq
    nbytes = tq.bitnet_chain_workspace_size(dims, 1)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    plan = tq.bitnet_chain_prepare(dims, [(blobs[0:7], norms_dev[0])], ws, nbytes)
    x = torch.from_numpy(inputs.chain_input(chain)).cuda()
    tq.bitnet_chain_run(plan, x)
    tq.bitnet_chain_status(plan)
    ws_ = [inputs.chain_projection(chain, 0, p) for p in range(7)]
    norms = [inputs.chain_norm(chain, 0, j) for j in range(4)]
    ref, _ = oracle.bitnet_layer(chain.dims(), [w["trits"][0] for w in ws_],
                                 np.array([w["scales"][0] for w in ws_], dtype=np.float32), norms,
                                 inputs.chain_input(chain))
    got = x.cpu().numpy()
    del plan, ws, x
    release_device()
    return {"layers": 1, "bit_exact": bool(np.array_equal(got.view(np.uint32), ref.view(np.uint32)))}


def chain_cpu_baseline(chain, seconds: float) -> dict:
    import oracle
    orc = oracle.default()
    ws_ = [inputs.chain_projection(chain, 0, p) for p in range(7)]
    trits = [w["trits"][0] for w in ws_]
    s_w = np.array([w["scales"][0] for w in ws_], dtype=np.float32)
    norms = [inputs.chain_norm(chain, 0, j) for j in range(4)]
    x = inputs.chain_input(chain)
    layer_bytes = chain_bytes(chain, 0) / chain.layers
    reps, t0 = 0, time.perf_counter()
    while True:
        orc.bitnet_layer(chain.dims(), trits, s_w, norms, x)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(layer_bytes * reps / el / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "layer 0 of the chain, %d repetitions, %.1f s (%.2f tokens/s over %d layers); C oracle, "
                      "one thread" % (reps, el, reps / el / chain.layers, chain.layers)}


def main_chain(args):
    import torch
    from ternary_weight_amd import tq
    chain = CHAINS["chain"]
    t_build = time.perf_counter()
    # the decode stack's packed projections are the chain's weights (same seeds and recipe)
    stack = Stack(CASES["cfg2"], 1, fused=False)
    assert len(stack.blobs) == 7 * chain.layers
    norms_dev = [[torch.from_numpy(inputs.chain_norm(chain, l, j)).cuda() for j in range(4)]
                 for l in range(chain.layers)]
    dims = tq.bitnet_dims(*chain.dims())
    nbytes = tq.bitnet_chain_workspace_size(dims, chain.layers)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    layers = [(stack.blobs[7 * l:7 * l + 7], norms_dev[l]) for l in range(chain.layers)]
    plan = tq.bitnet_chain_prepare(dims, layers, ws, nbytes, workgroups=args.workgroups)
    x0 = torch.from_numpy(inputs.chain_input(chain)).cuda()
    x = x0.clone()
    print("built chain: %d layers, %.1f MB packed, %d workgroups (%.1f s)"
          % (chain.layers, stack.blob_bytes / 1e6, plan.workgroups, time.perf_counter() - t_build),
          file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()
    spin_up(args.spin_up_ms)
    for _ in range(args.warmup):
        tq.bitnet_chain_run(plan, x)
    tq.bitnet_chain_status(plan)
    # timed region: K tokens, each through every layer (the state carries over
    # from token to token; the work does not depend on its values)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        tq.bitnet_chain_run(plan, x)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tq.bitnet_chain_status(plan)
    ms_step = start.elapsed_time(end) / args.steps
    gbytes = chain_bytes(chain, stack.blob_bytes)
    value = gbytes / (ms_step / 1e3) / 1e9
    ceiling = hbm_ceiling() if args.ceiling else None
    check = None if args.no_check else chain_spot_check(chain, stack.blobs, norms_dev, dims)
    cpu = None if args.no_cpu_baseline else chain_cpu_baseline(chain, args.cpu_seconds)
    kernel_name = "k_bitnet_chain"
    out = {
        "metric": METRIC_CHAIN,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic (seeded SplitMix64; the BitNet decode stack's weights, RMSNorm weights U[0.5, 1.5), "
                "x ~ N(0,1))",
        "config": {
            "workload": chain.name,
            "layers": chain.layers,
            "M": 1,
            "step": "one token through every layer: a reset launch and one cooperative launch (4 phases per layer; "
                    "a phase waits until the blocks it reads are written)",
            "packed_weight_bytes": stack.blob_bytes,
            "workgroups": plan.workgroups,
        },
        "tok_per_s": round(1e3 / ms_step, 1),
        "us_per_layer": round(ms_step * 1e3 / chain.layers, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(value, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(value / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(kernel_name),
            "kernel": kernel_name,
            "bytes_per_launch": gbytes,
        },
        "cpu_baseline": cpu,
        "hbm_ceiling": ceiling,
        "parity_spot_check": check,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(out), flush=True)
    # every launch complete and every buffer the plan points at released
    # before the interpreter exits
    tq.bitnet_chain_status(plan)
    del plan, ws, x, x0, layers, norms_dev, stack
    release_device()


# ---------------------------------------------------------------------------
# MoE experts: the routed experts of every layer for a decode batch.
# ---------------------------------------------------------------------------
def moe_reference(moe, layer, e, p, a, m, rows=None):
    """The oracle's outputs [m][len(rows)] of one problem of a MoeStack, from
    host-regenerated weights and activations."""
    import oracle
    h = inputs.moe_projection(moe, layer, e, p, rows=rows)
    toks, pairs = inputs.moe_expert_rows(moe, layer)[e]
    c = a - sum(len(t) for t, _ in inputs.moe_expert_rows(moe, layer)[:e])   # first token of the chunk
    src = inputs.moe_hidden(moe, layer)[toks[c:c + m]] if p < 2 else inputs.moe_inter(moe, layer)[pairs[c:c + m]]
    if moe.x_type == I8:
        q, s = oracle.act_quant_i8(src, F32)
        return oracle.gemv_i8(moe.planes, moe.group, moe.layout, h["trits"], h["scales"], q, s, None)["y64"]
    return oracle.gemv_fp(moe.planes, moe.group, moe.layout, h["trits"], h["scales"], src, moe.x_type, None)


def moe_spot_check(stack, n_prob=3, rows=64) -> dict:
    """Rows of a few problems (first, last, one between) against the oracle."""
    import torch
    torch.cuda.synchronize()
    rng = np.random.default_rng(98)
    picks = sorted({0, len(stack.meta) - 1, int(rng.integers(len(stack.meta)))})[:n_prob]
    worst = 0.0
    for i in picks:
        layer, e, p, a, m = stack.meta[i]
        n = stack.shapes[p][1]
        r = np.sort(rng.choice(n, size=min(rows, n), replace=False))
        y = stack.ys[layer][p][a:a + m].cpu().numpy()[:, r]
        worst = max(worst, rel_err(y, moe_reference(stack.moe, layer, e, p, a, m, rows=r)))
    return {"problems": len(picks), "rows_each": rows, "max_rel_err": worst}


def moe_cpu_baseline(stack, seconds: float) -> dict:
    """The oracle on the host cores over the routed experts of layer 0, in order."""
    import oracle
    moe = stack.moe
    threads = oracle_threads()
    orc = oracle.default()
    hid, inter = inputs.moe_hidden(moe, 0), inputs.moe_inter(moe, 0)
    route = inputs.moe_expert_rows(moe, 0)
    xsz = {BF16: 2, F32: 4, I8: 4}[moe.x_type]
    done, reps, experts, t0 = 0, 0, 0, time.perf_counter()
    el = 0.0
    for e in range(moe.experts):
        toks, pairs = route[e]
        if not len(toks):
            continue
        for p, (_, n, kin) in enumerate(stack.shapes):
            h = inputs.moe_projection(moe, 0, e, p)
            x = hid[toks] if p < 2 else inter[pairs]
            t1 = time.perf_counter()
            if moe.x_type == I8:
                q, s = orc.act_quant_i8(x, F32)
                orc.gemv_i8(moe.planes, moe.group, moe.layout, h["trits"], h["scales"], q, s, None, nthreads=threads)
            else:
                orc.gemv_fp(moe.planes, moe.group, moe.layout, h["trits"], h["scales"], x, moe.x_type, None,
                            nthreads=threads)
            el += time.perf_counter() - t1
            done += (moe.planes * n * kin // 4 + 2 * moe.planes * n * (kin // moe.group)
                     + len(toks) * kin * xsz + 4 * len(toks) * n)
            reps += 1
        experts += 1
        if el >= seconds:
            break
    return {"value": round(done / el / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "the first %d routed experts of layer 0 (gate, up, down each, their routed tokens), "
                      "%.1f s of oracle time (input generation excluded); C oracle, OpenMP over output rows"
                      % (experts, el)}


def main_moe(args):
    import torch
    from synth.configs import MOES
    import dataclasses
    moe = MOES["moe"]
    if args.batch:
        moe = dataclasses.replace(moe, batch=args.batch)
    moe = dataclasses.replace(moe, x_type={"i8": I8, "bf16": BF16, "f32": F32}[args.moe_x])
    if moe.x_type != I8:
        moe = dataclasses.replace(moe, name=moe.name.replace("int8 x (per-token absmax)", args.moe_x + " x"))
    t_build = time.perf_counter()
    stack = MoeStack(moe, fused=args.fused)
    stack.prepare(args.waves, args.row_blocks)
    print("built moe: %d layers x %d experts, %.1f GB packed, %d problems (%d routed experts), "
          "plan %d items x %d blocks x %d waves (%.1f s)"
          % (moe.layers, moe.experts, stack.blob_bytes / 1e9, len(stack.meta), stack.active_experts(),
             stack.plan.n_items, stack.plan.row_blocks, stack.plan.waves, time.perf_counter() - t_build),
          file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()
    spin_up(args.spin_up_ms)
    for _ in range(args.warmup):
        stack.quantize()
        stack.gemv()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        stack.quantize()
        stack.gemv()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / args.steps
    gemv_avg = ms_step
    if stack.quant:    # the product kernel alone, back to back between one pair of events
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(args.steps):
            stack.gemv()
        g1.record(stream)
        torch.cuda.synchronize()
        gemv_avg = g0.elapsed_time(g1) / args.steps
    gbytes = stack.gemv_bytes()
    value = (gbytes + stack.quant_bytes()) / (ms_step / 1e3) / 1e9
    achieved = gbytes / (gemv_avg / 1e3) / 1e9
    kernel_name = decode_kernel_name(stack.plan, stack.run_type, moe.layout, moe.planes, moe.group)
    ceiling = hbm_ceiling() if args.ceiling else None
    check = None if args.no_check else moe_spot_check(stack)
    cpu = None if args.no_cpu_baseline else moe_cpu_baseline(stack, args.cpu_seconds)
    out = {
        "metric": METRIC_MOE,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {I8: "i8", BF16: "bf16", F32: "f32"}[moe.x_type],
        "data": "synthetic (seeded SplitMix64; trits P(0)=0.4, x ~ N(0,1), uniform top-%d routing)" % moe.top_k,
        "config": {
            "workload": moe.name,
            "layers": moe.layers,
            "experts": moe.experts,
            "top_k": moe.top_k,
            "batch_tokens": moe.batch,
            "routed_experts": stack.active_experts(),
            "problems": len(stack.meta),
            "max_tokens_per_problem": stack.max_tokens,
            "planes": moe.planes,
            "group": moe.group,
            "step": ("act-quant of every layer's gathered rows (one launch) + " if stack.quant else "") +
                    "one grouped launch over every routed (layer, expert, projection) of the batch, each "
                    "with its own token count" + ("; fp32 inputs quantised per token to int8 inside it"
                                                  if stack.fused else ""),
            "packed_weight_bytes": stack.blob_bytes,
            "grouped_waves": stack.plan.waves,
            "grouped_row_blocks": stack.plan.row_blocks,
        },
        "tok_per_s_equiv": round(moe.batch * 1e3 / ms_step, 1),
        "gemv_us": round(gemv_avg * 1e3, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(kernel_name),
            "kernel": kernel_name,
            "bytes_per_launch": gbytes,
        },
        "cpu_baseline": cpu,
        "hbm_ceiling": ceiling,
        "parity_spot_check": check,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(out), flush=True)
    release_device()


# ---------------------------------------------------------------------------
# The ternarizer: fit the dense weights of one layer into planes (offline).
# ---------------------------------------------------------------------------
def main_ternarize(args):
    import torch
    import oracle
    from ternary_weight_amd import tq
    from synth.configs import LLAMA_8B
    codec = args.config == "ternarize_codec"
    K, g, layout = (3, 16, CODEBOOK) if codec else (3, 256, GROUP_F16)
    shapes = LLAMA_8B["proj"]
    cb = torch.from_numpy(gen.codebook_f16(inputs.N_CODEBOOK).view(np.int16)).cuda() if codec else None
    jobs = []
    for p, (name, n, kin) in enumerate(shapes):
        w = torch.empty((n, kin), dtype=torch.float32, device="cuda")
        device.fill(device.K_NORMAL_F32, gen.tensor_seed(9, 0, p, 7), 0, w)   # N(0, 1) dense weight
        d = tq.desc(K, g, layout, n, kin, n_codebook=inputs.N_CODEBOOK if codec else 0)
        trits = torch.empty((K, n, kin), dtype=torch.int8, device="cuda")
        scales = (torch.empty((n, kin // g), dtype=torch.uint8, device="cuda") if codec
                  else torch.empty((K, n, kin // g), dtype=torch.int16, device="cuda"))
        jobs.append((name, d, w, trits, scales))
    torch.cuda.synchronize()
    # weights of trained linears are ~N(0, 0.02^2); the fit is scale-equivariant up to the
    # codebook's range, so the codec is fed 0.02 w
    if codec:
        for j in jobs:
            j[2].mul_(0.02)

    def step():
        for name, d, w, trits, scales in jobs:
            tq.ternarize(d, w, trits, scales, cb)

    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    ceiling = hbm_ceiling() if args.ceiling else None
    weights = sum(n * kin for (_, n, kin) in shapes)
    # algorithmic bytes: the dense weight read once, the trits written once (int8), the scales
    scale_b = sum(n * (kin // g) * (1 if codec else 2 * K) for (_, n, kin) in shapes)
    nbytes = 4 * weights + K * weights + scale_b
    value = nbytes / (ms_step / 1e3) / 1e9
    check = None
    if not args.no_check:   # the first projection's first 256 rows against the oracle
        name, d, w, trits, scales = jobs[1]
        rows = w[:256].cpu().numpy()
        t_ref, s_ref = oracle.ternarize(K, g, layout, rows, gen.codebook_f16(inputs.N_CODEBOOK) if codec else None)
        # the 256-row fit of a row-wise method equals those rows of the full fit
        t = trits[:, :256].cpu().numpy()
        s = scales[:256].cpu().numpy() if codec else scales[:, :256].cpu().numpy().view(np.uint16)
        check = {"projection": name, "rows": 256,
                 "bit_exact": bool(np.array_equal(t, t_ref) and np.array_equal(s, s_ref))}
    out = {
        "metric": "ternarizer effective HBM GB/s (% of peak), Llama-3.1-8B-shaped layer",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic dense weights, seeded N(0,1)" + (" x 0.02" if codec else ""),
        "config": {"workload": "fit the 7 projections of one Llama-3.1-8B-shaped layer: " +
                               ("the d=3 codec, groups of 16, 27-entry codebook" if codec else
                                "K=3 greedy planes, f16 scale per group of 256"),
                   "weights": weights},
        "roofline": {"bound": "hbm", "achieved": round(value, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBS, 4),
                     "traffic": None,
                     "kernel": "k_tern_codec" if codec else "k_tern_group_lds", "bytes_per_step": nbytes,
                     "launches_per_step": len(jobs)},
        "hbm_ceiling": ceiling,
        "parity_spot_check": check,
    }
    print(json.dumps(out), flush=True)
    release_device()


if __name__ == "__main__":
    main()
