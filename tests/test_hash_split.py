"""The split of the keep hash that the HIP kernels evaluate (CPU only).

The keep word of query row i and key pair m = j / 2 is mix32(row + m), and
mix32 starts with a multiply, so the kernels distribute it over the sum:
(row + m) * C1 = row * C1 + m * C1 (mod 2^32). The forward and dQ kernels
form (row + 2*hi + k0/2) * C1 once per tile (k0 the tile's first key, hi the
lane's half of the wave) and add a compile-time pair offset times C1 per
pair, deciding the even key from the low and the odd key from the high 16
bits, both compared at the top of the word against T16 << 16. The dK/dV
kernel keeps row * C1 in LDS, adds (key / 2) * C1 of its lane and shifts its
half to the top. These tests check both rewritings against the oracle's
keep_halves / mix32 for tile bases at and beyond the 16-bit boundary and for
wrapping sums.
"""
import numpy as np
import pytest

from oracle.dropout_hash import dropout_keep, dropout_threshold, keep_halves, mix32, row_words

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
def test_tile_word_then_one_add_per_pair(bc):
    rng = np.random.default_rng(11)
    rows = [int(x) for x in rng.integers(0, 2**32, 48, dtype=np.uint64)] + [M32, M32 - 5]
    bases = [0, bc, 65536 - bc, 65536, 3 * 65536 + 7 * bc, 2**31 - bc]
    for r in rows:
        for hi in (0, 1):
            rw = (r + 2 * hi) & M32  # the lane half's 4*hi keys = 2*hi pairs folded into the row word
            for k0 in bases:
                y = ((rw + k0 // 2) * C1) & M32  # once per tile
                for kb in range(bc // 32):
                    for v in range(0, 16, 2):
                        off = kb * 16 + 4 * (v >> 2) + ((v & 3) >> 1)
                        u = _finish(y + ((off * C1) & M32))
                        for e in (0, 1):  # elements v (even key) and v + 1 (odd key)
                            key = k0 + kb * 32 + _crow(v + e, hi)
                            assert key % 2 == e
                            w = int(mix32(np.uint32((r + key // 2) & M32)))
                            assert u == w
                            half = (w >> 16) if e else (w & 0xFFFF)
                            top = u if e else (u << 16) & M32  # the kernels' compare operand
                            assert top >> 16 == half


def test_row_words_times_c1_stored():
    # dK/dV: lanes own a key; the rows' words come from LDS already times C1
    rng = np.random.default_rng(12)
    rows = np.concatenate([rng.integers(0, 2**32, 200, dtype=np.uint64), [M32]]).astype(np.uint64)
    keys = np.concatenate([np.arange(0, 300), rng.integers(0, 2**31, 300)]).astype(np.uint64)
    side = (rows * np.uint64(C1)) & np.uint64(M32)
    keyc = ((keys >> np.uint64(1)) * np.uint64(C1)) & np.uint64(M32)
    x = (side[:, None] + keyc[None, :]) & np.uint64(M32)
    x ^= x >> np.uint64(13)
    x = (x * np.uint64(0xC2B2AE35)) & np.uint64(M32)
    x ^= x >> np.uint64(16)
    want = mix32((rows[:, None] + (keys >> np.uint64(1))[None, :]).astype(np.uint32))
    np.testing.assert_array_equal(x.astype(np.uint32), want)
    # the lane's half moved to the top: even keys shift by 16, odd keys by 0
    sh = np.where(keys % 2 == 1, 0, 16).astype(np.uint64)
    top = (x << sh[None, :]) & np.uint64(M32)
    half = np.where((keys % 2 == 1)[None, :], want >> np.uint32(16), want & np.uint32(0xFFFF))
    np.testing.assert_array_equal((top >> np.uint64(16)).astype(np.uint32), half)


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9, 1e-9])
def test_top_compare_equals_the_16_bit_threshold(p):
    # keep iff half >= T16 is the same as (half << 16) >= (T16 << 16) on 32 bits
    seed, b, h = 0x5EED0003, 1, 4
    rows, cols = np.arange(0, 64), np.arange(1000, 1200)
    hv = keep_halves(seed, b, h, rows, cols).astype(np.uint64)
    th = np.uint64(dropout_threshold(p) << 16)
    np.testing.assert_array_equal((hv << np.uint64(16)) >= th, dropout_keep(seed, b, h, rows, cols, p))
    assert row_words(seed, b, h, [0]).dtype == np.uint32
