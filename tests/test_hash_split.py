"""The split of the keep hash that the HIP kernels evaluate (CPU only).

The kernels do not call fmix32 on every (row word, key) pair. They apply its
first step, x ^ (x >> 16), once per tile and then finish each key with one
XOR and the remaining steps. These tests check that rewriting against the
oracle's fmix32 over every offset of a tile, for tile bases at the 16-bit
boundary and beyond.
"""
import numpy as np
import pytest

from oracle.dropout_hash import fmix32

M32 = np.uint64(0xFFFFFFFF)


def _head(x):
    x = np.asarray(x, dtype=np.uint64)
    return x ^ (x >> np.uint64(16))


def _tail(x):
    x = np.asarray(x, dtype=np.uint64)
    x = (x * np.uint64(0x85EBCA6B)) & M32
    x ^= x >> np.uint64(13)
    x = (x * np.uint64(0xC2B2AE35)) & M32
    x ^= x >> np.uint64(16)
    return x


def _crow(v, hi):
    # key offset of MFMA accumulator element v in a 32-key block (lane half hi)
    return 8 * (v >> 2) + 4 * hi + (v & 3)


@pytest.mark.parametrize("bc", [32, 64])
def test_tile_word_then_one_xor_per_key(bc):
    rng = np.random.default_rng(11)
    rows = rng.integers(0, 2**32, 64, dtype=np.uint64)
    bases = np.array([0, bc, 65536 - bc, 65536, 3 * 65536 + 7 * bc, 2**31 - bc], dtype=np.uint64)
    for r in rows:
        for hi in (0, 1):
            rw = np.uint64(int(r) ^ (4 * hi))  # the lane half folded into the row word
            for k0 in bases:
                y = _head(rw ^ k0)
                for kb in range(bc // 32):
                    for v in range(16):
                        key = int(k0) + kb * 32 + _crow(v, hi)
                        off = kb * 32 + 8 * (v >> 2) + (v & 3)
                        assert int(_tail(y ^ np.uint64(off))) == int(fmix32(int(r) ^ key))


def test_row_words_with_head_step_stored():
    # dK/dV: lanes own a key, rows come from LDS with the head step applied
    rng = np.random.default_rng(12)
    rows = rng.integers(0, 2**32, 200, dtype=np.uint64)
    keys = np.concatenate([np.arange(0, 300), rng.integers(0, 2**31, 300)]).astype(np.uint64)
    got = _tail(_head(rows)[:, None] ^ _head(keys)[None, :])
    want = np.array([[fmix32(int(r) ^ int(k)) for k in keys] for r in rows], dtype=np.uint64)
    np.testing.assert_array_equal(got, want)
