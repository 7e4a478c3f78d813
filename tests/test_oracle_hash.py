"""Pins of the oracle's dropout keep bits (CPU only)."""
import json
import math
import os

import numpy as np
import pytest

from oracle.dropout_hash import dropout_keep, dropout_threshold, fmix32, head_key

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
    assert dropout_threshold(0.1) == 429496729  # float32 0.1 would give 429496736
    assert dropout_threshold(0.5) == 2**31
    assert dropout_threshold(np.nextafter(1.0, 0.0)) == 2**32 - 1
    with pytest.raises(ValueError):
        dropout_threshold(1.0)
    with pytest.raises(ValueError):
        dropout_threshold(-0.1)


def _scalar_keep(seed, b, h, i, j, p):
    """Keep bit from the stated definition, one element at a time."""
    lo, hi = seed & M32, (seed >> 32) & M32
    k = fmix32((lo + 0x9E3779B9) & M32)
    for word in (hi, b, h):
        k = fmix32(k ^ word)
    x = (fmix32(k ^ i) + j) & M32
    x = (x * 0x85EBCA6B) & M32
    x ^= x >> 13
    x = (x * 0xC2B2AE35) & M32
    x ^= x >> 16
    return x >= math.floor(p * 2.0**32)


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
    sigma = math.sqrt(p * (1 - p) / n)
    assert abs(frac - (1 - p)) < 6 * sigma
    # per-row counts: chi-square against Binomial(1024, 0.9)
    rows = z.sum(axis=1)
    e, var = 1024 * (1 - p), 1024 * p * (1 - p)
    chi2 = ((rows - e) ** 2 / var).sum()
    assert abs(chi2 - 1024) < 6 * math.sqrt(2 * 1024)
    cols = z.sum(axis=0)
    chi2c = ((cols - e) ** 2 / var).sum()
    assert abs(chi2c - 1024) < 6 * math.sqrt(2 * 1024)
    # two heads agree on a fraction ~ p^2 + (1-p)^2
    z2 = dropout_keep(0x5EED0003, 1, 3, np.arange(1024), np.arange(1024), p)
    agree = (z == z2).mean()
    ex = p * p + (1 - p) ** 2
    assert abs(agree - ex) < 6 * math.sqrt(ex * (1 - ex) / n)


def test_neighbouring_keys_and_rows_are_uncorrelated():
    # the key index enters by addition, so check that adjacent keys of a row,
    # adjacent rows at one key, and the anti-diagonal neighbour agree only at
    # the rate of independent bits, p^2 + (1-p)^2
    for p in (0.1, 0.5):
        z = dropout_keep(0x5EED0003, 0, 7, np.arange(1025), np.arange(1025), p)
        ex = p * p + (1 - p) ** 2
        for a, b in ((z[:, 1:], z[:, :-1]), (z[1:, :], z[:-1, :]), (z[1:, :-1], z[:-1, 1:])):
            agree = (a == b).mean()
            assert abs(agree - ex) < 6 * math.sqrt(ex * (1 - ex) / a.size), (p, agree, ex)


def test_large_indices_wrap_as_uint32():
    # indices near 2^14 and beyond behave like any other counter value
    z = dropout_keep(99, 0, 0, np.arange(16380, 16390), np.arange(16380, 16390), 0.5)
    for a, i in enumerate(range(16380, 16390)):
        for c, j in enumerate(range(16380, 16390)):
            assert z[a, c] == _scalar_keep(99, 0, 0, i, j, 0.5)
