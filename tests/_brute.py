"""Independent brute-force attention for tiny inputs (pure Python, mpmath).

Written from the definition of softmax attention, element by element, with
no numpy matrix products and no code shared with ``oracle/``. Used only to
pin the oracle on tiny inputs.
"""
from __future__ import annotations

import math

import mpmath

M32 = 0xFFFFFFFF


def _fmix(x: int) -> int:
    # MurmurHash3 finalizer, scalar Python ints (its constants are pinned by
    # the published MurmurHash3 vectors in test_oracle_hash.py)
    x &= M32
    x ^= x >> 16
    x = (x * 0x85EBCA6B) & M32
    x ^= x >> 13
    x = (x * 0xC2B2AE35) & M32
    x ^= x >> 16
    return x


def keep_bit(seed: int, b: int, h: int, i: int, j: int, p: float) -> bool:
    if p == 0.0:
        return True
    k = _fmix(((seed & M32) + 0x9E3779B9) & M32)
    k = _fmix(k ^ ((seed >> 32) & M32))
    k = _fmix(k ^ b)
    k = _fmix(k ^ h)
    # keys 2m and 2m+1 share one word: the pair index is added to the row
    # word, the finalizer runs from its first multiply on (its leading shift
    # left out), and the key takes the low (even j) or high (odd j) 16 bits
    x = (_fmix(k ^ i) + j // 2) & M32
    x = (x * 0x85EBCA6B) & M32
    x ^= x >> 13
    x = (x * 0xC2B2AE35) & M32
    u = x ^ (x >> 16)
    half = (u >> 16) if j % 2 else (u & 0xFFFF)
    return half >= math.floor(p * 65536.0)


def is_valid(i: int, j: int, causal: bool, block_mask, mask_block: int) -> bool:
    if causal and j > i:
        return False
    if block_mask is not None and not block_mask[i // mask_block][j // mask_block]:
        return False
    return True


def brute_forward(q, k, v, scale, causal=False, block_mask=None, mask_block=1,
                  p=0.0, seed=0, b=0, h=0, dps=50):
    """q, k, v: nested lists (N x d) of floats. Returns (O, LSE) as lists of
    mpmath numbers (LSE = -inf for a row with no valid key)."""
    mpmath.mp.dps = dps
    N, d = len(q), len(q[0])
    O, L = [], []
    for i in range(N):
        s = {}
        for j in range(len(k)):
            if is_valid(i, j, causal, block_mask, mask_block):
                s[j] = mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[i][c]) * mpmath.mpf(k[j][c]) for c in range(d))
        if not s:
            O.append([mpmath.mpf(0)] * len(v[0]))
            L.append(-mpmath.inf)
            continue
        m = max(s.values())
        lse = m + mpmath.log(mpmath.fsum(mpmath.exp(x - m) for x in s.values()))
        row = []
        for c in range(len(v[0])):
            acc = []
            for j, x in s.items():
                if keep_bit(seed, b, h, i, j, p):
                    acc.append(mpmath.exp(x - lse) * mpmath.mpf(v[j][c]) / (1 - mpmath.mpf(p)))
            row.append(mpmath.fsum(acc))
        O.append(row)
        L.append(lse)
    return O, L


def brute_loss_grad_check_inputs(N, d, seed):
    import random

    r = random.Random(seed)
    mk = lambda: [[r.gauss(0, 1) for _ in range(d)] for _ in range(N)]  # noqa: E731
    return mk(), mk(), mk(), mk()
