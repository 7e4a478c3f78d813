"""Counter-based dropout keep bits (oracle side; test infrastructure only).

The pages put dropout between the softmax and the second matrix product in
the fused step list (FlashAttention milestone page, section "The idea", the
paragraph on the single kernel; inferensys glossary, "Kernel Fusion") but do
not say how the random bits are drawn. This library defines them as a
counter-based hash of (seed, b, h, i, j), so forward and backward regenerate
the same mask without storing it. One 32-bit word serves two neighbouring
keys: key 2m reads its low 16 bits and key 2m+1 its high 16 bits.

    fmix32(x)  : x ^= x >> 16; x *= 0x85EBCA6B; x ^= x >> 13;
                 x *= 0xC2B2AE35; x ^= x >> 16          (all mod 2^32)
    mix32(x)   : fmix32 without its first step:
                 x *= 0x85EBCA6B; x ^= x >> 13; x *= 0xC2B2AE35; x ^= x >> 16
    key(b, h)  = fmix32(fmix32(fmix32(fmix32(lo(seed) + 0x9E3779B9) ^ hi(seed)) ^ b) ^ h)
    row(i)     = fmix32(key ^ i)
    w(i, m)    = mix32(row(i) + m)                      (sum mod 2^32)
    half(i, j) = (w(i, floor(j / 2)) >> (16 * (j mod 2))) mod 2^16
    keep(i, j) = half(i, j) >= T16,   T16 = floor(p * 2^16) evaluated in float64

``fmix32`` is the finalizer of Austin Appleby's MurmurHash3 (public domain);
``mix32(x ^ (x >> 16)) == fmix32(x)`` ties the two. The pair index enters by
addition ahead of the first multiply, so the product
(row(i) + m) * 0x85EBCA6B splits into a per-row and a per-pair term; the row
word is already a full fmix32 output, so the first shift of fmix32 is left
out. A kept element has probability 1 - T16 / 2^16, which lies within 2^-16
of 1 - p; the surviving values are scaled by 1 / (1 - p) all the same.

Because w depends on i only through row(i) + m, two rows whose row words
differ by a small delta (|delta| < N/2) draw the same words shifted by delta
pairs: their keep masks agree after a shift of 2 * delta keys. Over the
N^2/2 row pairs of a head about N^3 / 2^33 are such pairs (1 at N = 2048,
about 500 at N = 16384).

The oracle's copy is written here with numpy uint32 arithmetic and shares
nothing with the GPU side.
"""
from __future__ import annotations

import math

import numpy as np

_M32 = 0xFFFFFFFF


def fmix32(x):
    """MurmurHash3 32-bit finalizer on a numpy uint32 array (or Python int)."""
    scalar = not isinstance(x, np.ndarray)
    a = np.atleast_1d(np.asarray(x, dtype=np.uint64) & np.uint64(_M32)).astype(np.uint32)
    a ^= a >> np.uint32(16)
    a = a * np.uint32(0x85EBCA6B)
    a ^= a >> np.uint32(13)
    a = a * np.uint32(0xC2B2AE35)
    a ^= a >> np.uint32(16)
    return int(a[0]) if scalar else a


def mix32(x):
    """fmix32 without its first xor-shift, on numpy uint32 values (any shape)."""
    x = np.asarray(x, dtype=np.uint32)
    a = np.atleast_1d(x).copy()  # array arithmetic wraps mod 2^32 without warnings
    a = a * np.uint32(0x85EBCA6B)
    a ^= a >> np.uint32(13)
    a = a * np.uint32(0xC2B2AE35)
    a ^= a >> np.uint32(16)
    return a.reshape(x.shape)


def head_key(seed: int, b: int, h: int) -> int:
    """Per-(b, h) hash key from the 64-bit seed."""
    lo = seed & _M32
    hi = (seed >> 32) & _M32
    k = fmix32((lo + 0x9E3779B9) & _M32)
    k = fmix32(k ^ hi)
    k = fmix32(k ^ (b & _M32))
    k = fmix32(k ^ (h & _M32))
    return k


def row_words(seed: int, b: int, h: int, rows) -> np.ndarray:
    """row(i) = fmix32(key(b, h) ^ i) for the given query rows (uint32)."""
    rows = np.asarray(rows, dtype=np.int64)
    return fmix32(rows.astype(np.uint32) ^ np.uint32(head_key(seed, b, h)))


def dropout_threshold(p: float) -> int:
    """Threshold T16 = floor(p * 2^16) in float64; keep iff the 16-bit half >= T16."""
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must lie in [0, 1)")
    return int(math.floor(float(p) * 65536.0))


def keep_halves(seed: int, b: int, h: int, rows, cols) -> np.ndarray:
    """The 16-bit value half(i, j) that decides key j of query row i (uint32
    array ``[len(rows)][len(cols)]``, values below 2^16)."""
    cols = np.asarray(cols, dtype=np.int64)
    r = row_words(seed, b, h, rows)
    w = mix32(r[:, None] + (cols // 2).astype(np.uint32)[None, :])  # uint32 sum wraps mod 2^32
    shift = (np.uint32(16) * (cols % 2).astype(np.uint32))[None, :]
    return (w >> shift) & np.uint32(0xFFFF)


def dropout_keep(seed: int, b: int, h: int, rows, cols, p: float) -> np.ndarray:
    """Keep bits for query rows ``rows`` x key columns ``cols`` of head (b, h).

    Returns a bool array ``[len(rows)][len(cols)]``; all True when p == 0.
    """
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    if p == 0.0:
        return np.ones((rows.size, cols.size), dtype=bool)
    return keep_halves(seed, b, h, rows, cols) >= np.uint32(dropout_threshold(p))
