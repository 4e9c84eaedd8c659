"""The device copy of the input generator reproduces the host one bit for bit."""
import numpy as np
import pytest

from synth import device, gen, inputs
from synth.configs import CASES
from tests.gpu_util import host, torch

pytestmark = pytest.mark.gpu


def test_device_generator_matches_host():
    t = torch()
    seed, start, n = 0xABCDEF12345, 777, 100003
    for kind, hostf, dtype in [
        (device.K_TRITS, lambda: gen.trits(seed, start, n), t.int8),
        (device.K_DIGITS, lambda: gen.digits(seed, start, n), t.int8),
        (device.K_INDICES, lambda: gen.indices(seed, start, n, 27), t.uint8),
        (device.K_NORMAL_F64, lambda: gen.normal(seed, start, n), t.float64),
        (device.K_NORMAL_F32, lambda: gen.normal(seed, start, n).astype(np.float32), t.float32),
        (device.K_NORMAL_BF16, lambda: gen.bf16_bits(gen.normal(seed, start, n)).view(np.int16), t.int16),
    ]:
        out = t.empty(n, dtype=dtype, device="cuda")
        device.fill(kind, seed, start, out, a=27.0)
        t.cuda.synchronize()
        want = hostf()
        got = host(out)
        assert np.array_equal(got.view(np.uint8), np.ascontiguousarray(want).view(np.uint8)), kind
    lo, span = gen.log_uniform_params(1e-3, 1e-1)
    for div in (1.0, 3.0, 9.0):
        out = t.empty(n, dtype=t.int16, device="cuda")
        device.fill(device.K_LOGU_F16, seed, start, out, a=lo, b=span, div=div)
        t.cuda.synchronize()
        want = gen.f16_bits(gen.log_uniform(seed, start, n, 1e-3, 1e-1) / div)
        assert np.array_equal(host(out).view(np.uint16), want)
    out = t.empty(n, dtype=t.float32, device="cuda")
    device.fill(device.K_LOGU_F32, seed, start, out, a=lo, b=span)
    t.cuda.synchronize()
    assert np.array_equal(host(out), gen.log_uniform(seed, start, n, 1e-3, 1e-1).astype(np.float32))


@pytest.mark.parametrize("name", ["cfg1", "cfg2", "cfg3", "cfg4"])
def test_device_projection_matches_host(name):
    case = CASES[name]
    N, Kin = (256, 512) if name == "cfg1" else (128, 512)
    d = device.projection(case, 2, 3, N, Kin, M=3 if name == "cfg4" else None)
    h = inputs.projection(case, 2, 3, N, Kin, M=3 if name == "cfg4" else None)
    torch().cuda.synchronize()
    assert np.array_equal(host(d["trits"]), h["trits"])
    assert np.array_equal(host(d["scales"]).view(h["scales"].dtype), h["scales"])
    assert np.array_equal(host(d["x"]).view(h["x"].dtype), h["x"])
