"""The compact base-3 codec layout (TQ_SCALE_CODEBOOK_B3) without a GPU:
the test-side reader of the documented stream against an encoder written
here from the same description, exhaustively over all 729 pair codes; the
blob size in closed form; descriptor validation."""
from __future__ import annotations

import itertools

import numpy as np
import pytest

from tests.gpu_util import b3_digits, b3_stream_codes
from ternary_weight_amd import tq


def _encode_pair(v0, v1):
    return (v0 % 27) + 27 * (v1 % 27)


def _stream_words(codes):
    """32 ten-bit codes -> ten little-endian dwords (code j at bits 10j..10j+9)."""
    big = 0
    for j, c in enumerate(codes):
        assert 0 <= c < 1024
        big |= int(c) << (10 * j)
    return np.array([(big >> (32 * i)) & 0xFFFFFFFF for i in range(10)], dtype=np.uint32)


def test_every_pair_code_round_trips():
    # the 27 balanced-ternary values of three digits, plane 0 the most significant
    vals = {}
    for t0, t1, t2 in itertools.product((-1, 0, 1), repeat=3):
        vals[9 * t0 + 3 * t1 + t2] = (t0, t1, t2)
    assert sorted(vals) == list(range(-13, 14))              # a bijection onto [-13, 13]
    codes = [_encode_pair(a, b) for a in range(-13, 14) for b in range(-13, 14)]
    assert sorted(codes) == list(range(729))                  # every code below 729, once
    assert _encode_pair(0, 0) == 0                            # padding (zero bytes) is two zero weights
    d = b3_digits(np.array(codes))                            # [3][729][2]
    k = 0
    for a in range(-13, 14):
        for b in range(-13, 14):
            assert tuple(d[:, k, 0]) == vals[a] and tuple(d[:, k, 1]) == vals[b]
            k += 1
    # codes never written read as zeros
    assert not b3_digits(np.arange(729, 1024)).any()


def test_stream_bit_positions():
    rng = np.random.default_rng(3)
    for _ in range(50):
        codes = rng.integers(0, 1024, size=32)
        got = b3_stream_codes(_stream_words(codes)[None, :])[0]
        assert np.array_equal(got, codes)
    # field 3 straddles dwords 0 and 1 (bits 30..39)
    w = _stream_words([0, 0, 0, 0x3FF] + [0] * 28)
    assert w[0] == 0xC0000000 and w[1] == 0xFF


def _size(N, Kin, g=16):
    return tq.packed_size(tq.desc(3, g, tq.SCALE_CODEBOOK_B3, N, Kin, n_codebook=27))


def _align(v):
    return (v + 255) // 256 * 256


@pytest.mark.parametrize("N,Kin,g", [(64, 64, 16), (4096, 4096, 16), (14336, 4096, 16), (100, 80, 16),
                                     (4096, 14336, 32), (1, 16, 16)])
def test_packed_size_closed_form(N, Kin, g):
    NB, NC, G = (N + 63) // 64, (Kin + 63) // 64, Kin // g
    NID = (G + 5) // 6
    codes = NB * NC * 2560                   # 40 bytes per row and 64 columns: 5 bits per weight
    want = _align(256 + codes) + 256 + NB * NID * 256
    assert _size(N, Kin, g) == _align(want)
    old = tq.packed_size(tq.desc(3, g, tq.SCALE_CODEBOOK, N, Kin, n_codebook=27))
    assert _size(N, Kin, g) < old             # the two-bit planes take 6 bits per weight


def test_bits_per_weight_at_llama_shapes():
    # 5 bits per weight of codes, plus the group indices (six to a dword), one
    # bit per weight below the two-bit planes' codec
    N, Kin = 14336, 4096
    bpw = 8 * _size(N, Kin) / (N * Kin)
    G = Kin // 16
    assert abs(bpw - (5 + 32 * ((G + 5) // 6) / Kin)) < 1e-3
    old = 8 * tq.packed_size(tq.desc(3, 16, tq.SCALE_CODEBOOK, N, Kin, n_codebook=27)) / (N * Kin)
    assert abs(old - bpw - 1.0) < 1e-3


def test_descriptor_rules():
    with pytest.raises(tq.TQError) as e:
        tq.packed_size(tq.desc(2, 16, tq.SCALE_CODEBOOK_B3, 64, 64, n_codebook=27))
    assert e.value.status == tq.ERR_UNSUPPORTED
    with pytest.raises(tq.TQError) as e:
        tq.packed_size(tq.desc(3, 16, tq.SCALE_CODEBOOK_B3, 64, 64, n_codebook=0))
    assert e.value.status == tq.ERR_ARG
    with pytest.raises(tq.TQError) as e:
        tq.packed_size(tq.desc(3, 24, tq.SCALE_CODEBOOK_B3, 64, 96, n_codebook=27))
    assert e.value.status == tq.ERR_ARG
    with pytest.raises(tq.TQError):
        tq.packed_size(tq.desc(3, 16, 4, 64, 64, n_codebook=27))
