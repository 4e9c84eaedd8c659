"""Host generator: SplitMix64 streams and the draws built on them.

Every draw is counter based: element ``i`` of the stream with seed ``s`` is
``mix64(s + (i + 1) * GAMMA)`` -- exactly the (i+1)-th output of SplitMix64
(Steele, Lea & Flood, "Fast splittable pseudorandom number generators",
OOPSLA 2014) started from state ``s``.  Any slice of any tensor can therefore
be regenerated on its own, which is what lets the tests check sampled rows of
full-size problems without materialising the whole input on the host.

Floating-point draws use only IEEE basic operations (+ - * /, floor and exact
bit manipulation) in a fixed order, with no fused multiply-add, so that the
device copy of this generator (``synth_kernels.hip``, compiled with
``-ffp-contract=off``) reproduces them bit for bit.  The transcendental
functions needed by Box-Muller and the log-uniform draw are therefore written
out here (series after exact range reduction) rather than taken from libm.
Their accuracy (~1e-15 relative) only matters for the shape of the
distribution; determinism is what the tests rely on.

Recipes (one line each; the workloads' own text fixes the distributions):
  uniform      u = (r >> 11) * 2^-53                              in [0, 1)
  trit         u < 0.3 -> -1,  u < 0.6 -> +1,  else 0             P(0) = 0.4
  digit        floor(3u) - 1                                      uniform {-1,0,1}
  index        floor(n u)                                         uniform {0..n-1}
  normal       Box-Muller, element i uses draws 2i and 2i+1:
               sqrt(-2 ln(1 - u_a)) * cos(2 pi u_b)
  log-uniform  exp(ln a + u (ln b - ln a))
  f16          round-to-nearest-even from the fp64 draw
  bf16         fp64 -> fp32 (RNE) -> bf16 (RNE)
"""
from __future__ import annotations

import numpy as np

U64 = np.uint64
GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1

# Seed base: the ASCII bytes of "trits".
SEED_BASE = 0x7472697473


def mix64_int(z: int) -> int:
    """SplitMix64 output function on a Python int (reference scalar form)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * _M1) & MASK64
    z = ((z ^ (z >> 27)) * _M2) & MASK64
    return z ^ (z >> 31)


def tensor_seed(cfg: int, layer: int, proj: int, kind: int) -> int:
    """Seed of one tensor of one workload: a SplitMix64 output of the packed ids."""
    key = SEED_BASE ^ (cfg << 48) ^ (layer << 32) ^ (proj << 16) ^ kind
    return mix64_int((key + GAMMA) & MASK64)


def _mix64(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = (z ^ (z >> U64(30))) * U64(_M1)
        z = (z ^ (z >> U64(27))) * U64(_M2)
    return z ^ (z >> U64(31))


def stream(seed: int, start: int, count: int) -> np.ndarray:
    """Outputs ``start .. start+count-1`` (0-based) of SplitMix64 seeded with ``seed``."""
    i = np.arange(start + 1, start + count + 1, dtype=U64)
    with np.errstate(over="ignore"):
        z = U64(seed & MASK64) + i * U64(GAMMA)
    return _mix64(z)


def _u01(r: np.ndarray) -> np.ndarray:
    return (r >> U64(11)).astype(np.float64) * (2.0 ** -53)


def uniform(seed: int, start: int, count: int) -> np.ndarray:
    return _u01(stream(seed, start, count))


def trits(seed: int, start: int, count: int) -> np.ndarray:
    """int8 trits with P(-1) = P(+1) = 0.3 and P(0) = 0.4."""
    u = uniform(seed, start, count)
    out = np.zeros(count, dtype=np.int8)
    out[u < 0.6] = 1
    out[u < 0.3] = -1
    return out


def digits(seed: int, start: int, count: int) -> np.ndarray:
    """int8 digits uniform over {-1, 0, +1}."""
    u = uniform(seed, start, count)
    return (np.floor(u * 3.0) - 1.0).astype(np.int8)


def indices(seed: int, start: int, count: int, n: int) -> np.ndarray:
    """uint8 indices uniform over {0 .. n-1}."""
    u = uniform(seed, start, count)
    return np.floor(u * float(n)).astype(np.uint8)


# ---------------------------------------------------------------------------
# Deterministic elementary functions (basic IEEE operations only).
# ---------------------------------------------------------------------------
LN2 = float.fromhex("0x1.62e42fefa39efp-1")
LN2_HI = float.fromhex("0x1.62e42fee00000p-1")
LN2_LO = float.fromhex("0x1.a39ef35793c76p-33")
INV_LN2 = float.fromhex("0x1.71547652b82fep+0")
SQRT2 = float.fromhex("0x1.6a09e667f3bcdp+0")
HALF_PI = float.fromhex("0x1.921fb54442d18p+0")

N_LN = 14      # terms of 2 atanh(s) = ln m
N_TRIG = 14    # terms of the sin / cos series
N_EXP = 22     # terms of the exp series
N_SQRT = 7     # Newton steps


def _ln_coeffs() -> list:
    return [1.0 / float(2 * k + 1) for k in range(N_LN)]


def _cos_coeffs() -> list:
    c = [1.0]
    for k in range(1, N_TRIG):
        c.append(c[-1] / (-float((2 * k - 1) * (2 * k))))
    return c


def _sin_coeffs() -> list:
    c = [1.0]
    for k in range(1, N_TRIG):
        c.append(c[-1] / (-float((2 * k) * (2 * k + 1))))
    return c


def _exp_coeffs() -> list:
    c = [1.0]
    for k in range(1, N_EXP):
        c.append(c[-1] / float(k))
    return c


LN_C = _ln_coeffs()
COS_C = _cos_coeffs()
SIN_C = _sin_coeffs()
EXP_C = _exp_coeffs()


def det_ln(u: np.ndarray) -> np.ndarray:
    """ln(u) for positive normal fp64 u: u = m 2^e, ln m = 2 atanh((m-1)/(m+1))."""
    u = np.asarray(u, dtype=np.float64)
    bits = u.view(U64)
    e = ((bits >> U64(52)) & U64(0x7FF)).astype(np.int64) - 1023
    m = ((bits & U64(0x000FFFFFFFFFFFFF)) | U64(0x3FF0000000000000)).view(np.float64)
    big = m > SQRT2
    m = np.where(big, m * 0.5, m)
    e = np.where(big, e + 1, e)
    s = (m - 1.0) / (m + 1.0)
    s2 = s * s
    p = np.full_like(s, LN_C[N_LN - 1])
    for k in range(N_LN - 2, -1, -1):
        p = p * s2 + LN_C[k]
    return e.astype(np.float64) * LN2 + (2.0 * s) * p


def det_cos2pi(u: np.ndarray) -> np.ndarray:
    """cos(2 pi u) for u in [0, 1), reduced exactly by quarter turns."""
    u = np.asarray(u, dtype=np.float64)
    v = u * 4.0
    q = np.floor(v)
    f = v - q
    flip = f > 0.5
    g = np.where(flip, 1.0 - f, f)
    x = g * HALF_PI
    x2 = x * x
    c = np.full_like(x, COS_C[N_TRIG - 1])
    for k in range(N_TRIG - 2, -1, -1):
        c = c * x2 + COS_C[k]
    s = np.full_like(x, SIN_C[N_TRIG - 1])
    for k in range(N_TRIG - 2, -1, -1):
        s = s * x2 + SIN_C[k]
    s = s * x
    cf = np.where(flip, s, c)
    sf = np.where(flip, c, s)
    qi = q.astype(np.int64)
    return np.select([qi == 0, qi == 1, qi == 2], [cf, -sf, -cf], sf)


def det_sqrt(y: np.ndarray) -> np.ndarray:
    """sqrt(y), y >= 0: Newton from a power of two at or above the root."""
    y = np.asarray(y, dtype=np.float64)
    bits = y.view(U64)
    e = ((bits >> U64(52)) & U64(0x7FF)).astype(np.int64) - 1023
    h = (e + 2) // 2
    x = ((h + 1023).astype(U64) << U64(52)).view(np.float64)
    pos = y > 0.0
    ysafe = np.where(pos, y, 1.0)
    x = np.where(pos, x, 1.0)
    for _ in range(N_SQRT):
        x = 0.5 * (x + ysafe / x)
    return np.where(pos, x, 0.0)


def det_exp(z: np.ndarray) -> np.ndarray:
    """exp(z) for |z| < 700: z = k ln2 + r (Cody-Waite), series for e^r, times 2^k."""
    z = np.asarray(z, dtype=np.float64)
    k = np.floor(z * INV_LN2 + 0.5)
    r = (z - k * LN2_HI) - k * LN2_LO
    p = np.full_like(r, EXP_C[N_EXP - 1])
    for j in range(N_EXP - 2, -1, -1):
        p = p * r + EXP_C[j]
    scale = ((k.astype(np.int64) + 1023).astype(U64) << U64(52)).view(np.float64)
    return p * scale


def normal(seed: int, start: int, count: int) -> np.ndarray:
    """fp64 N(0,1) by Box-Muller; element i consumes stream outputs 2i and 2i+1."""
    r = stream(seed, 2 * start, 2 * count)
    ua = _u01(r[0::2])
    ub = _u01(r[1::2])
    rad = det_sqrt(-2.0 * det_ln(1.0 - ua))
    return rad * det_cos2pi(ub)


def log_uniform_params(a: float, b: float) -> tuple:
    la = float(det_ln(np.array([a]))[0])
    lb = float(det_ln(np.array([b]))[0])
    return la, lb - la


def log_uniform(seed: int, start: int, count: int, a: float, b: float) -> np.ndarray:
    lo, span = log_uniform_params(a, b)
    u = uniform(seed, start, count)
    return det_exp(lo + u * span)


# ---------------------------------------------------------------------------
# Storage rounding.
# ---------------------------------------------------------------------------
def f16_bits(v: np.ndarray) -> np.ndarray:
    """fp64 -> IEEE binary16 bits, round to nearest even."""
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def f32_to_bf16_bits(v32: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bits, round to nearest even (inputs are finite)."""
    u = np.asarray(v32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> U64(16)) & U64(1)
    return ((u + U64(0x7FFF) + lsb) >> U64(16)).astype(np.uint16)


def bf16_bits(v: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 (RNE) -> bf16 (RNE)."""
    return f32_to_bf16_bits(np.asarray(v, dtype=np.float64).astype(np.float32))


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


def codebook_f16(n: int = 27, lo: float = 1e-4, hi: float = 1e-1) -> np.ndarray:
    """n log-spaced values from lo to hi, endpoints included, as f16 bits."""
    j = np.arange(n, dtype=np.float64)
    v = lo * (hi / lo) ** (j / float(n - 1))
    return f16_bits(v)
