"""The test-side reader of the blob layout, pinned by hand-worked examples
of the documented bit positions (no GPU)."""
import numpy as np

from tests.gpu_util import read_blob


def test_reader_bit_positions():
    K, N, Kin = 2, 70, 80      # two row blocks, two column chunks
    NB, NC = 2, 2
    raw = np.zeros(256 + NB * NC * K * 1024 + 256, dtype=np.uint8)
    words = raw[256:256 + NB * NC * K * 1024].view(np.uint32).reshape(NB, NC, K, 64, 4)
    # row 0, plane 0: column 16*0 + 4*2 + 1 = 9 -> code 01 in byte 1, bits 4..5
    words[0, 0, 0, 0, 0] |= np.uint32(1 << (8 * 1 + 2 * 2))
    # row 65 (block 1, lane 1), plane 1, column 64 + 16*3 + 4*3 + 2 = 126 -> code 10 in byte 2, bits 6..7
    words[1, 1, 1, 1, 3] |= np.uint32(2 << (8 * 2 + 2 * 3))
    # row 5, plane 0, column 30 = 16*1 + 4*3 + 2 -> code 11 (reads as 0)
    words[0, 0, 0, 5, 1] |= np.uint32(3 << (8 * 2 + 2 * 3))
    raw[256 + NB * NC * K * 1024:][:4] = np.array([0.25], np.float32).view(np.uint8)
    out = read_blob(raw, K, N, Kin, 0)
    t = out["trits"]
    assert t.shape == (2, 70, 80)
    assert t[0, 0, 9] == 1
    nz = np.argwhere(t != 0)
    assert sorted(map(tuple, nz.tolist())) == [(0, 0, 9)]       # column 126 is beyond Kin = 80
    assert out["codes"][1, 65, 126] == 2 and out["codes"][0, 5, 30] == 3
    assert out["scales"][0] == np.float32(0.25)


def test_reader_group_scales_and_indices():
    K, N, Kin, g = 1, 64, 256, 64      # G = 4 groups -> 2 pair dwords
    raw = np.zeros(256 + 4 * 1024 + 2 * 256, dtype=np.uint8)
    end = 256 + 4 * 1024
    sw = raw[end:end + 2 * 256].view(np.uint32).reshape(1, 2, 1, 64)
    sw[0, 1, 0, 7] = np.uint32(0x3C00 | (0x4000 << 16))        # row 7: group 2 = 1.0, group 3 = 2.0
    out = read_blob(raw, K, N, Kin, 1, g)
    assert out["scales"][0, 7, 2] == 0x3C00 and out["scales"][0, 7, 3] == 0x4000
    # codebook: 6 five-bit indices per dword
    K, N, Kin, g = 3, 64, 128, 16       # G = 8 -> 2 index dwords
    raw = np.zeros(256 + 2 * 3 * 1024 + 256 + 2 * 256, dtype=np.uint8)
    end = 256 + 2 * 3 * 1024
    raw[end:end + 2] = np.array([0x068E], np.uint16).view(np.uint8)
    iw = raw[end + 256:end + 256 + 512].view(np.uint32).reshape(1, 2, 64)
    iw[0, 0, 3] = np.uint32((26 << 25) | (1 << 5))              # row 3: group 5 = 26, group 1 = 1
    iw[0, 1, 3] = np.uint32(9 << 5)                              # row 3: group 7 = 9
    out = read_blob(raw, K, N, Kin, 2, g)
    assert out["scales"][3].tolist() == [0, 1, 0, 0, 0, 26, 0, 9]
    assert out["codebook"][0] == 0x068E
