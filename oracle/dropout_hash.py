"""Counter-based dropout keep bits (oracle side; test infrastructure only).

The pages put dropout between the softmax and the second matrix product in
the fused step list (FlashAttention milestone page, section "The idea", the
paragraph on the single kernel; inferensys glossary, "Kernel Fusion") but do
not say how the random bits are drawn. This library defines them as a
counter-based hash of (seed, b, h, i, j), so forward and backward regenerate
the same mask without storing it:

    fmix32(x)  : x ^= x >> 16; x *= 0x85EBCA6B; x ^= x >> 13;
                 x *= 0xC2B2AE35; x ^= x >> 16          (all mod 2^32)
    mix32(x)   : fmix32 without its first step:
                 x *= 0x85EBCA6B; x ^= x >> 13; x *= 0xC2B2AE35; x ^= x >> 16
    key(b, h)  = fmix32(fmix32(fmix32(fmix32(lo(seed) + 0x9E3779B9) ^ hi(seed)) ^ b) ^ h)
    row(i)     = fmix32(key ^ i)
    u(i, j)    = mix32(row(i) + j)                      (sum mod 2^32)
    keep(i, j) = u(i, j) >= T,   T = floor(p * 2^32) evaluated in float64

``fmix32`` is the finalizer of Austin Appleby's MurmurHash3 (public domain).
The key index enters by addition ahead of the first multiply, so the
product (row(i) + j) * 0x85EBCA6B splits into a per-row and a per-key term;
the row word is already a full fmix32 output, so the first shift of fmix32
is left out. The oracle's copy is written here with numpy uint32 arithmetic
and shares nothing with the GPU side.
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


def dropout_threshold(p: float) -> int:
    """Integer threshold T = floor(p * 2^32) in float64; keep iff hash >= T."""
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must lie in [0, 1)")
    return int(math.floor(float(p) * 4294967296.0))


def dropout_keep(seed: int, b: int, h: int, rows, cols, p: float) -> np.ndarray:
    """Keep bits for query rows ``rows`` x key columns ``cols`` of head (b, h).

    Returns a bool array ``[len(rows)][len(cols)]``; all True when p == 0.
    """
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    if p == 0.0:
        return np.ones((rows.size, cols.size), dtype=bool)
    T = dropout_threshold(p)
    k = np.uint32(head_key(seed, b, h))
    r = fmix32((rows.astype(np.uint32) ^ k))
    u = mix32(r[:, None] + cols.astype(np.uint32)[None, :])  # uint32 sum wraps mod 2^32
    return u >= np.uint32(T)
