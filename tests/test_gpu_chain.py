"""The decode chain (tq_bitnet_chain_*) against the CPU oracle, bit for bit.

Each layer's q, k, v and the hidden state after the last layer are compared
with oracle.bitnet_layer on the same seeded inputs (layer l's q, k and v
are a function of the state entering it, so every layer's state is pinned):
the small BitNet-shaped chain over all its layers and several grid sizes
(items per workgroup and column splits change with the grid), a chain whose
widths are not multiples of the 64-row block, and the BitNet b1.58-2B shapes
over all 30 layers at the default grid and another, each run repeated on
the same plan.  The only rounding that the two sides take in a different
order is the fp64 sum of squares inside RMSNorm (see tq.h); a mismatch
there would show as a difference in the last bits of one layer.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from synth import inputs
from synth.configs import CHAINS

pytestmark = pytest.mark.gpu


def _device_layers(chain, n_layers):
    import torch
    from ternary_weight_amd import tq
    keep, layers, host = [], [], []
    for layer in range(n_layers):
        blobs, trits, s_w = [], [], []
        for p, (_, N, Kin) in enumerate(chain.proj_shapes()):
            w = inputs.chain_projection(chain, layer, p)
            d = tq.desc(1, 0, tq.SCALE_TENSOR, N, Kin)
            blob = torch.empty(tq.packed_size(d), dtype=torch.uint8, device="cuda")
            t = torch.from_numpy(w["trits"]).cuda()
            s = torch.from_numpy(w["scales"]).cuda()
            tq.pack(d, t, s, None, blob)
            keep += [t, s]
            blobs.append(blob)
            trits.append(w["trits"][0])
            s_w.append(w["scales"][0])
        norms_h = [inputs.chain_norm(chain, layer, j) for j in range(4)]
        norms = [torch.from_numpy(n).cuda() for n in norms_h]
        layers.append((blobs, norms))
        host.append((trits, np.array(s_w, dtype=np.float32), norms_h))
    torch.cuda.synchronize()
    return layers, host, keep


def _device_layers_generated(chain, n_layers):
    """As _device_layers, with the weights drawn by the device copy of the
    seeded generator (equal to the host one, test_gpu_synth) and copied back
    for the oracle: the host generator is too slow for 30 full-size layers."""
    import torch
    from synth import device
    from synth.configs import CASES
    from ternary_weight_amd import tq
    wcase = CASES["cfg2"]
    assert chain.weights_cfg == wcase.cfg
    layers, host = [], []
    for layer in range(n_layers):
        blobs, trits, s_w = [], [], []
        for p, (_, N, Kin) in enumerate(chain.proj_shapes()):
            d = device.projection(wcase, layer, p, N, Kin, M=1)
            desc = tq.desc(1, 0, tq.SCALE_TENSOR, N, Kin)
            blob = torch.empty(tq.packed_size(desc), dtype=torch.uint8, device="cuda")
            tq.pack(desc, d["trits"], d["scales"], None, blob)
            blobs.append(blob)
            trits.append(d["trits"][0].cpu().numpy())
            s_w.append(float(d["scales"][0].cpu().numpy()))
            del d
        norms_h = [inputs.chain_norm(chain, layer, j) for j in range(4)]
        layers.append((blobs, [torch.from_numpy(n).cuda() for n in norms_h]))
        host.append((trits, np.array(s_w, dtype=np.float32), norms_h))
    torch.cuda.synchronize()
    return layers, host


def _oracle_chain(chain, host):
    x = inputs.chain_input(chain)
    xs, qkvs = [], []
    for trits, s_w, norms in host:
        x, qkv = oracle.bitnet_layer(chain.dims(), trits, s_w, norms, x)
        xs.append(x.copy())
        qkvs.append(qkv)
    return xs, qkvs


def _run(chain, layers, n_layers, workgroups=0):
    import torch
    from ternary_weight_amd import tq
    dims = tq.bitnet_dims(*chain.dims())
    nbytes = tq.bitnet_chain_workspace_size(dims, n_layers)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    plan = tq.bitnet_chain_prepare(dims, layers[:n_layers], ws, nbytes, workgroups=workgroups)
    x = torch.from_numpy(inputs.chain_input(chain)).cuda()
    nqkv = (chain.n_heads + 2 * chain.n_kv) * chain.head_dim
    qkv = torch.zeros((n_layers, nqkv), dtype=torch.float32, device="cuda")
    tq.bitnet_chain_run(plan, x, qkv)
    tq.bitnet_chain_status(plan)
    return plan, ws, x.cpu().numpy(), qkv.cpu().numpy()


@pytest.fixture(scope="module")
def small():
    chain = CHAINS["chain_small"]
    layers, host, keep = _device_layers(chain, chain.layers)
    xs, qkvs = _oracle_chain(chain, host)
    return chain, layers, xs, qkvs, keep


@pytest.mark.parametrize("workgroups", [0, 1, 7, 64])
def test_small_chain_matches_oracle(small, workgroups):
    chain, layers, xs, qkvs, _ = small
    print("chain_small layers=%d workgroups=%d" % (chain.layers, workgroups), flush=True)
    plan, _, x, qkv = _run(chain, layers, chain.layers, workgroups)
    if workgroups:
        assert plan.workgroups == workgroups
    for layer in range(chain.layers):
        assert np.array_equal(qkv[layer].view(np.uint32), qkvs[layer].view(np.uint32)), layer
    assert np.array_equal(x.view(np.uint32), xs[-1].view(np.uint32))


def test_small_chain_prefixes_and_repeats(small):
    """Shorter chains give the oracle's intermediate states; a second run on
    the same workspace (whose accumulators the first left cleared) repeats
    the first bit for bit."""
    import torch
    from ternary_weight_amd import tq
    chain, layers, xs, qkvs, _ = small
    for n in (1, 2):
        plan, ws, x, _ = _run(chain, layers, n)
        assert np.array_equal(x.view(np.uint32), xs[n - 1].view(np.uint32)), n
    x2 = torch.from_numpy(inputs.chain_input(chain)).cuda()
    tq.bitnet_chain_run(plan, x2)
    tq.bitnet_chain_status(plan)
    assert np.array_equal(x2.cpu().numpy().view(np.uint32), xs[1].view(np.uint32))


def _check_runs(chain, layers, xs, qkvs, n_layers, workgroups, repeats):
    import torch
    from ternary_weight_amd import tq
    plan, ws, x, qkv = _run(chain, layers, n_layers, workgroups)
    for r in range(repeats):
        if r:
            xd = torch.from_numpy(inputs.chain_input(chain)).cuda()
            qd = torch.zeros_like(torch.from_numpy(qkv)).cuda()
            tq.bitnet_chain_run(plan, xd, qd)
            tq.bitnet_chain_status(plan)
            x, qkv = xd.cpu().numpy(), qd.cpu().numpy()
        for layer in range(n_layers):
            assert np.array_equal(qkv[layer].view(np.uint32), qkvs[layer].view(np.uint32)), \
                (workgroups, r, layer)
        assert np.array_equal(x.view(np.uint32), xs[n_layers - 1].view(np.uint32)), (workgroups, r)
    del plan, ws


@pytest.mark.parametrize("workgroups", [0, 3, 16, 97])
def test_ragged_widths_chain(workgroups):
    """hidden 240, 48-wide KV heads, FFN 720: every projection ends in a
    partly padded 64-row block, whose accumulator rows must not reach the
    next block's."""
    chain = CHAINS["chain_ragged"]
    print("chain_ragged layers=%d workgroups=%d" % (chain.layers, workgroups), flush=True)
    layers, host, keep = _device_layers(chain, chain.layers)
    xs, qkvs = _oracle_chain(chain, host)
    _check_runs(chain, layers, xs, qkvs, chain.layers, workgroups, repeats=3)


@pytest.fixture(scope="module")
def bitnet30():
    chain = CHAINS["chain"]
    print("chain BitNet-2B: generating %d layers" % chain.layers, flush=True)
    layers, host = _device_layers_generated(chain, chain.layers)
    xs, qkvs = _oracle_chain(chain, host)
    return chain, layers, xs, qkvs


@pytest.mark.parametrize("workgroups", [0, 97, 256])
def test_bitnet_shapes_all_layers(bitnet30, workgroups):
    """Every one of the 30 BitNet b1.58-2B layers, bit for bit, three runs on one plan."""
    chain, layers, xs, qkvs = bitnet30
    print("chain BitNet-2B layers=%d workgroups=%d" % (chain.layers, workgroups), flush=True)
    _check_runs(chain, layers, xs, qkvs, chain.layers, workgroups, repeats=3)


def test_prepare_rejects_mismatched_blobs(small):
    import torch
    from ternary_weight_amd import tq
    chain, layers, _, _, _ = small
    dims = tq.bitnet_dims(*chain.dims())
    nbytes = tq.bitnet_chain_workspace_size(dims, 1)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    blobs, norms = layers[0]
    swapped = [blobs[0], blobs[1], blobs[2], blobs[3], blobs[6], blobs[5], blobs[4]]   # gate <-> down
    with pytest.raises(tq.TQError) as e:
        tq.bitnet_chain_prepare(dims, [(swapped, norms)], ws, nbytes)
    assert e.value.status == tq.ERR_SHAPE
    with pytest.raises(tq.TQError):
        tq.bitnet_chain_prepare(dims, [(blobs, norms)], ws, nbytes - 256)
    with pytest.raises(tq.TQError) as e:
        tq.bitnet_chain_prepare(dims, [(blobs, norms)], ws, nbytes, workgroups=1 << 20)
    assert e.value.status == tq.ERR_UNSUPPORTED
