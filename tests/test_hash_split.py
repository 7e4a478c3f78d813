"""The split of the keep hash that the HIP kernels evaluate (CPU only).

The keep word is mix32(row + key), and mix32 starts with a multiply, so the
kernels distribute it over the sum: (row + key) * C1 = row * C1 + key * C1
(mod 2^32). The forward and dQ kernels form (row + tile base) * C1 once per
tile and add a compile-time off * C1 per key; the dK/dV kernel keeps
row * C1 in LDS and adds key * C1 of its lane. These tests check both
rewritings against the oracle's mix32 for tile bases at and beyond the
16-bit boundary and for wrapping sums.
"""
import numpy as np
import pytest

from oracle.dropout_hash import mix32

M32 = 0xFFFFFFFF
C1 = 0x85EBCA6B


def _finish(x):
    # the steps of mix32 after its first multiply
    x &= M32
    x ^= x >> 13
    x = (x * 0xC2B2AE35) & M32
    x ^= x >> 16
    return x


def _crow(v, hi):
    # key offset of MFMA accumulator element v in a 32-key block (lane half hi)
    return 8 * (v >> 2) + 4 * hi + (v & 3)


@pytest.mark.parametrize("bc", [32, 64])
def test_tile_word_then_one_add_per_key(bc):
    rng = np.random.default_rng(11)
    rows = [int(x) for x in rng.integers(0, 2**32, 48, dtype=np.uint64)] + [M32, M32 - 5]
    bases = [0, bc, 65536 - bc, 65536, 3 * 65536 + 7 * bc, 2**31 - bc]
    for r in rows:
        for hi in (0, 1):
            rw = (r + 4 * hi) & M32  # the lane half's key offset folded into the row word
            for k0 in bases:
                y = ((rw + k0) * C1) & M32  # once per tile
                for kb in range(bc // 32):
                    for v in range(16):
                        key = k0 + kb * 32 + _crow(v, hi)
                        off = kb * 32 + 8 * (v >> 2) + (v & 3)
                        got = _finish(y + ((off * C1) & M32))
                        assert got == int(mix32(np.uint32((r + key) & M32)))


def test_row_words_times_c1_stored():
    # dK/dV: lanes own a key; the rows' words come from LDS already times C1
    rng = np.random.default_rng(12)
    rows = np.concatenate([rng.integers(0, 2**32, 200, dtype=np.uint64), [M32]]).astype(np.uint64)
    keys = np.concatenate([np.arange(0, 300), rng.integers(0, 2**31, 300)]).astype(np.uint64)
    side = (rows * np.uint64(C1)) & np.uint64(M32)
    keyc = (keys * np.uint64(C1)) & np.uint64(M32)
    x = (side[:, None] + keyc[None, :]) & np.uint64(M32)
    x ^= x >> np.uint64(13)
    x = (x * np.uint64(0xC2B2AE35)) & np.uint64(M32)
    x ^= x >> np.uint64(16)
    want = mix32((rows[:, None] + keys[None, :]).astype(np.uint32))
    np.testing.assert_array_equal(x.astype(np.uint32), want)
