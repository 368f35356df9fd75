"""The device byte layout of packed codes (include/moeq.h) is a pure
re-layout of the oracle's packing: the test helpers that map between the two
invert each other, and the field order yields the natural code pairs the
decode kernels rely on.  CPU only."""
import numpy as np

import oracle
from tests.gpu_util import CHUNK_CODES, FIELD_CODE, device_codes, device_packed, device_sz


def test_relayout_round_trip():
    rng = np.random.default_rng(12)
    for bits in (4, 6, 8):
        q = rng.integers(0, 2 ** bits, (128, 192)).astype(np.uint8)
        dev = device_packed(q, bits)
        assert dev.size == oracle.pack(q, bits).size
        assert np.array_equal(device_codes(dev, 128, 192, bits), q)


def test_field_order_gives_natural_pairs():
    """4-bit: (dword >> 4j) & 0x000F000F of chunk dword d must hold codes
    8d + 2j and 8d + 2j + 1; 6-bit: the field pairs the unpacking combines,
    (0,3) (1,4) (5,8) (6,9) (10,13) (11,14) (2,7) (12,15), hold codes
    (2p, 2p + 1)."""
    for bits in (4, 6, 8):
        assert sorted(FIELD_CODE[bits]) == list(range(CHUNK_CODES[bits]))
    q = np.arange(32, dtype=np.uint8).reshape(1, 32) % 16
    codes = np.tile(np.arange(32, dtype=np.uint8) % 16, (64, 2))        # 64 rows x 64 codes
    dev = device_packed(codes, 4).reshape(2, 64, 16)                     # [chunk][row][16 B]
    words = dev[0, 0].view(np.uint32)                                    # row 0, chunk 0
    for d in range(4):
        for j in range(4):
            lo, hi = (int(words[d]) >> (4 * j)) & 0xF, (int(words[d]) >> (4 * j + 16)) & 0xF
            assert (lo, hi) == ((8 * d + 2 * j) % 16, (8 * d + 2 * j + 1) % 16)
    lo6 = [0, 1, 5, 6, 10, 11, 2, 12]
    hi6 = [3, 4, 8, 9, 13, 14, 7, 15]
    for p in range(8):
        assert (FIELD_CODE[6][lo6[p]], FIELD_CODE[6][hi6[p]]) == (2 * p, 2 * p + 1)


def test_sz_relayout():
    w = np.arange(128 * 3, dtype=np.uint32).reshape(128, 3)
    d = device_sz(w)
    # group g of row r at ((r // 64) * 3 + g) * 64 + r % 64
    for r in (0, 5, 63, 64, 127):
        for g in range(3):
            assert d[((r // 64) * 3 + g) * 64 + r % 64] == w[r, g]
