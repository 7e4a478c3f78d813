"""Pins of the oracle's dropout keep bits (CPU only)."""
import json
import math
import os

import numpy as np
import pytest

from oracle.dropout_hash import dropout_keep, dropout_threshold, fmix32, head_key, keep_halves, mix32, row_words

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "murmur3_x86_32_vectors.json")
M32 = 0xFFFFFFFF


def _rotl(x, r):
    return ((x << r) | (x >> (32 - r))) & M32


def _murmur3_x86_32(data: bytes, seed: int) -> int:
    """MurmurHash3_x86_32 body (block mix, tail, length) around the oracle's fmix32."""
    c1, c2 = 0xCC9E2D51, 0x1B873593
    h = seed & M32
    nblocks = len(data) // 4
    for i in range(nblocks):
        k = int.from_bytes(data[4 * i:4 * i + 4], "little")
        k = _rotl((k * c1) & M32, 15)
        h ^= (k * c2) & M32
        h = (_rotl(h, 13) * 5 + 0xE6546B64) & M32
    tail = data[4 * nblocks:]
    k = 0
    if len(tail) >= 3:
        k ^= tail[2] << 16
    if len(tail) >= 2:
        k ^= tail[1] << 8
    if len(tail) >= 1:
        k ^= tail[0]
        k = _rotl((k * c1) & M32, 15)
        h ^= (k * c2) & M32
    h ^= len(data)
    return fmix32(h)


def test_fmix32_published_murmur3_vectors():
    vecs = json.load(open(GOLDEN))["vectors"]
    assert len(vecs) >= 10
    for hexbytes, seed, expect in vecs:
        assert _murmur3_x86_32(bytes.fromhex(hexbytes), seed) == int(expect, 16), (hexbytes, seed)


def test_fmix32_vectorized_matches_scalar():
    xs = np.random.default_rng(1).integers(0, 2**32, size=1000, dtype=np.uint64).astype(np.uint32)
    vec = fmix32(xs)
    for x, y in zip(xs[:50], vec[:50]):
        assert fmix32(int(x)) == int(y)


def test_fmix32_is_a_bijection_on_a_slice():
    # fmix32 is invertible, so distinct inputs give distinct outputs
    xs = np.arange(1 << 18, dtype=np.uint32) * np.uint32(2654435761)
    assert np.unique(fmix32(xs)).size == xs.size


def test_threshold_is_computed_in_float64():
    assert dropout_threshold(0.0) == 0
    assert dropout_threshold(0.1) == 6553  # floor(6553.6)
    assert dropout_threshold(0.5) == 2**15
    assert dropout_threshold(np.nextafter(1.0, 0.0)) == 2**16 - 1
    assert dropout_threshold(1.0 / 65536) == 1
    assert dropout_threshold(np.nextafter(1.0 / 65536, 0.0)) == 0
    with pytest.raises(ValueError):
        dropout_threshold(1.0)
    with pytest.raises(ValueError):
        dropout_threshold(-0.1)


def test_mix32_is_fmix32_after_its_first_shift():
    # ties mix32 to the vector-pinned fmix32: fmix32(x) = mix32(x ^ (x >> 16))
    rng = np.random.default_rng(3)
    xs = rng.integers(0, 2**32, size=1_200_000, dtype=np.uint64).astype(np.uint32)
    edges = np.array([0, 1, 2**16 - 1, 2**16, 2**16 + 1, 2**31 - 1, 2**31, 2**32 - 2, 2**32 - 1], dtype=np.uint32)
    xs = np.concatenate([xs, edges])
    np.testing.assert_array_equal(mix32(xs ^ (xs >> np.uint32(16))), fmix32(xs))
    # and mix32 is the Python-int fmix32 of the same pre-shifted word on a few values
    for x in [0, 1, 0xDEADBEEF, 2**32 - 1]:
        assert int(mix32(np.uint32(x ^ (x >> 16)))) == fmix32(x)


def test_head_key_and_row_words_are_fmix32_chains():
    # the per-(b, h) key and the row word, built step by step from the
    # vector-pinned fmix32 (Python ints, one call per step)
    for seed in (0, 1, 0x5EED0003, 0x0123456789ABCDEF, 2**64 - 1):
        for b, h in ((0, 0), (3, 15), (1, 7), (2**31, 2**32 - 1)):
            k0 = fmix32(((seed & M32) + 0x9E3779B9) & M32)
            k1 = fmix32(k0 ^ (seed >> 32))
            k2 = fmix32(k1 ^ b)
            k3 = fmix32(k2 ^ h)
            assert head_key(seed, b, h) == k3, (seed, b, h)
            rows = np.array([0, 1, 4095, 16383, 65535], dtype=np.int64)
            want = [fmix32(k3 ^ int(i)) for i in rows]
            assert row_words(seed, b, h, rows).tolist() == want


def test_a_rows_pair_words_are_distinct():
    # mix32 is a bijection and the pair index is added to a fixed row word,
    # so the N/2 words of a row (one per key pair) are all distinct
    for seed, b, h, i in ((0x5EED0003, 0, 0, 0), (7, 3, 15, 16383), (2**64 - 1, 1, 2, 2**20)):
        r = row_words(seed, b, h, [i])[0]
        m = np.arange(2**17, dtype=np.uint32)
        w = mix32(r + m)
        assert np.unique(w).size == m.size


def test_halves_are_the_low_and_high_bits_of_one_word():
    seed, b, h = 0x5EED0003, 2, 9
    rows = np.array([0, 5, 4096])
    cols = np.arange(0, 40)
    hv = keep_halves(seed, b, h, rows, cols)
    w = mix32(row_words(seed, b, h, rows)[:, None] + (cols[None, 0::2] // 2).astype(np.uint32))
    np.testing.assert_array_equal(hv[:, 0::2], w & np.uint32(0xFFFF))
    np.testing.assert_array_equal(hv[:, 1::2], w >> np.uint32(16))
    # keep iff half >= T16, on both sides of the threshold
    for p in (0.1, 0.5, 0.9):
        z = dropout_keep(seed, b, h, rows, cols, p)
        np.testing.assert_array_equal(z, hv >= dropout_threshold(p))


def _scalar_keep(seed, b, h, i, j, p):
    """Keep bit from the stated definition, one element at a time."""
    lo, hi = seed & M32, (seed >> 32) & M32
    k = fmix32((lo + 0x9E3779B9) & M32)
    for word in (hi, b, h):
        k = fmix32(k ^ word)
    x = (fmix32(k ^ i) + j // 2) & M32
    x = (x * 0x85EBCA6B) & M32
    x ^= x >> 13
    x = (x * 0xC2B2AE35) & M32
    x ^= x >> 16
    half = x >> 16 if j % 2 else x & 0xFFFF
    return half >= math.floor(p * 2.0**16)


def test_keep_bits_follow_the_stated_chain():
    seed = 0x0123456789ABCDEF
    z = dropout_keep(seed, 3, 5, np.arange(20), np.arange(30), 0.37)
    for i in range(20):
        for j in range(30):
            assert z[i, j] == _scalar_keep(seed, 3, 5, i, j, 0.37)
    # the per-(b,h) key uses both halves of the seed, b and h
    assert len({head_key(seed, 0, 0), head_key(seed ^ (1 << 40), 0, 0), head_key(seed, 1, 0),
                head_key(seed, 0, 1)}) == 4


def test_p_zero_keeps_everything():
    assert dropout_keep(7, 0, 0, np.arange(64), np.arange(64), 0.0).all()


def test_keep_fraction_and_row_independence():
    p = 0.1
    z = dropout_keep(0x5EED0003, 1, 2, np.arange(1024), np.arange(1024), p)
    n = z.size
    frac = z.mean()
    q = dropout_threshold(p) / 65536.0  # drop probability of one 16-bit half
    sigma = math.sqrt(q * (1 - q) / n)
    assert abs(frac - (1 - q)) < 6 * sigma
    assert abs(q - p) < 2.0**-16
    # per-row counts: chi-square against Binomial(1024, 1 - q)
    rows = z.sum(axis=1)
    e, var = 1024 * (1 - q), 1024 * q * (1 - q)
    chi2 = ((rows - e) ** 2 / var).sum()
    assert abs(chi2 - 1024) < 6 * math.sqrt(2 * 1024)
    cols = z.sum(axis=0)
    chi2c = ((cols - e) ** 2 / var).sum()
    assert abs(chi2c - 1024) < 6 * math.sqrt(2 * 1024)
    # two heads agree on a fraction ~ q^2 + (1-q)^2
    z2 = dropout_keep(0x5EED0003, 1, 3, np.arange(1024), np.arange(1024), p)
    agree = (z == z2).mean()
    ex = q * q + (1 - q) ** 2
    assert abs(agree - ex) < 6 * math.sqrt(ex * (1 - ex) / n)


def test_neighbouring_keys_and_rows_are_uncorrelated():
    # the pair index enters by addition, so check that the two keys of one
    # word, the keys of neighbouring words, adjacent rows at one key and the
    # anti-diagonal neighbour agree only at the rate of independent bits
    for p in (0.1, 0.5):
        z = dropout_keep(0x5EED0003, 0, 7, np.arange(1025), np.arange(1026), p)
        q = dropout_threshold(p) / 65536.0
        ex = q * q + (1 - q) ** 2
        pairs = ((z[:, 0::2], z[:, 1::2]),      # low and high half of one word
                 (z[:, 1:-1:2], z[:, 2::2]),    # high half of word m, low half of word m+1
                 (z[:, 0:-2:2], z[:, 2::2]),    # low halves of neighbouring words
                 (z[1:, :], z[:-1, :]),         # adjacent rows
                 (z[1:, :-1], z[:-1, 1:]),      # anti-diagonal neighbours
                 (z[2:, :-2], z[:-2, 2:]))      # anti-diagonal, one word over
        for a, b in pairs:
            agree = (a == b).mean()
            assert abs(agree - ex) < 6 * math.sqrt(ex * (1 - ex) / a.size), (p, agree, ex)


def test_shifted_copy_rows_occur_at_the_stated_rate():
    # w depends on the row only through row(i) + m, so rows whose row words
    # differ by |delta| < N/2 draw the same words shifted by delta pairs.
    # Expected count over the N(N-1)/2 row pairs: N^2/2 * N / 2^32 = N^3 / 2^33.
    seed, N = 0x5EED0003, 4096
    counts = []
    for (b, h) in [(b, h) for b in range(4) for h in range(16)]:
        r = np.sort(row_words(seed, b, h, np.arange(N)).astype(np.int64))
        # circular differences of the sorted words (mod 2^32), all pairs closer than N/2
        ext = np.concatenate([r, r[:N] + 2**32])
        close = 0
        for lag in range(1, 8):
            close += int((ext[lag:lag + N] - ext[:N] < N // 2).sum())
        counts.append(close)
    mean = float(np.mean(counts))
    expect = N ** 3 / 2**33
    # Poisson count per head with mean 8 at N = 4096; 64 heads
    assert abs(mean - expect) < 6 * math.sqrt(expect / len(counts)), (mean, expect)
    # and such a pair really has shifted-copy masks
    b, h = 0, 0
    rw = row_words(seed, b, h, np.arange(N)).astype(np.int64)
    order = np.argsort(rw)
    gaps = np.diff(rw[order])
    k = int(np.argmin(gaps))
    i1, i2 = int(order[k]), int(order[k + 1])
    delta = int(rw[i2] - rw[i1])
    if delta < N // 2:
        cols = np.arange(0, N - 2 * delta)
        z1 = dropout_keep(seed, b, h, [i1], cols + 2 * delta, 0.5)
        z2 = dropout_keep(seed, b, h, [i2], cols, 0.5)
        np.testing.assert_array_equal(z1, z2)


def test_large_indices_wrap_as_uint32():
    # indices near 2^14 and beyond behave like any other counter value
    z = dropout_keep(99, 0, 0, np.arange(16380, 16390), np.arange(16380, 16390), 0.5)
    for a, i in enumerate(range(16380, 16390)):
        for c, j in enumerate(range(16380, 16390)):
            assert z[a, c] == _scalar_keep(99, 0, 0, i, j, 0.5)
