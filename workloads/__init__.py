"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and arranges them into the shapes of
the workloads. It holds none of the attention arithmetic, so both the fp64
oracle (under ``oracle/``) and the HIP path can be fed from it without sharing
any computation.

Workloads (the five shapes the attention pages are measured on):

* ``C1`` single head, non-causal forward, fp32:   B=1 H=1  N=128   d=64
* ``C2`` GPT-2-medium attention layer, causal:    B=8 H=16 N=1024  d=64  bf16
* ``C3`` training-style, causal, dropout p=0.1:   B=4 H=16 N=4096  d=64  bf16
* ``C4`` long context, causal, keys scaled x2:    B=1 H=32 N=16384 d=128 bf16
* ``C5`` block-sparse (128x128 blocks), dense:    B=2 H=16 N=8192  d=64  bf16

Recipe: one CPU ``torch.Generator`` per workload, seeded ``1000 + k`` for
workload ``Ck``; ``randn`` fp32 in the order Q, K, V, dO, each ``[B][H][N][d]``;
C4 multiplies K by 2 (a power of two, so exact); then a round-to-nearest-even
cast to the workload's dtype. The dropout key is ``0x5EED0003``. The C5 block
mask keeps the band ``(r, r)`` and ``(r, r-1)`` and every other block where
``numpy.random.default_rng(5005).random((64, 64))[r, c] < 0.1``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

DROPOUT_SEED = 0x5EED0003

_DTYPES = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str  # "fp32" | "bf16" | "fp16"
    causal: bool
    dropout_p: float = 0.0
    k_scale: float = 1.0
    block_sparse: bool = False
    mask_block: int = 128
    backward: bool = True
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self) -> torch.dtype:
        return _DTYPES[self.dtype]

    @property
    def dropout_seed(self) -> int:
        return DROPOUT_SEED if self.dropout_p > 0 else 0


WORKLOADS = {
    "C1": Workload("C1", 1, 1, 128, 64, "fp32", causal=False, backward=False, seed=1001),
    "C2": Workload("C2", 8, 16, 1024, 64, "bf16", causal=True, seed=1002),
    "C3": Workload("C3", 4, 16, 4096, 64, "bf16", causal=True, dropout_p=0.1, seed=1003),
    "C4": Workload("C4", 1, 32, 16384, 128, "bf16", causal=True, k_scale=2.0, seed=1004),
    "C5": Workload("C5", 2, 16, 8192, 64, "bf16", causal=False, block_sparse=True, seed=1005),
}

# Number of kept 128x128 blocks in the C5 mask (64 x 64 block grid).
C5_KEPT_BLOCKS = 518


def draw_qkvdo(B: int, H: int, N: int, d: int, dtype: torch.dtype, seed: int,
               k_scale: float = 1.0, with_do: bool = True):
    """Draw Q, K, V (and dO) ~ N(0,1) in fp32 from ``seed``, then cast to ``dtype``.

    Returns CPU tensors ``[B][H][N][d]``, contiguous. ``k_scale`` multiplies K
    before the cast (use powers of two to keep it exact).
    """
    g = torch.Generator().manual_seed(seed)
    shape = (B, H, N, d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    do = torch.randn(shape, generator=g, dtype=torch.float32) if with_do else None
    if k_scale != 1.0:
        k = k * k_scale
    q, k, v = (t.to(dtype).contiguous() for t in (q, k, v))
    if do is not None:
        do = do.to(dtype).contiguous()
    return q, k, v, do


def band_random_block_mask(nb: int, rng_seed: int = 5005, frac: float = 0.1) -> np.ndarray:
    """Block mask ``[nb][nb]`` (uint8, 1 = keep): band ``(r,r)``, ``(r,r-1)`` plus
    independent Bernoulli(``frac``) off-band blocks from ``default_rng(rng_seed)``."""
    u = np.random.default_rng(rng_seed).random((nb, nb))
    m = (u < frac).astype(np.uint8)
    r = np.arange(nb)
    m[r, r] = 1
    m[r[1:], r[1:] - 1] = 1
    return m


def random_block_mask(nb: int, seed: int, frac: float = 0.3, keep_diag: bool = True) -> np.ndarray:
    """A seeded random block mask for small tests; optionally keeps the diagonal."""
    m = (np.random.default_rng(seed).random((nb, nb)) < frac).astype(np.uint8)
    if keep_diag:
        m[np.arange(nb), np.arange(nb)] = 1
    return m


def workload_inputs(w: Workload, with_do: Optional[bool] = None):
    """Inputs of a named workload: dict with q, k, v, do (CPU tensors) and block_mask."""
    if with_do is None:
        with_do = w.backward
    q, k, v, do = draw_qkvdo(w.B, w.H, w.N, w.d, w.torch_dtype, w.seed, w.k_scale, with_do)
    bm = None
    if w.block_sparse:
        nb = (w.N + w.mask_block - 1) // w.mask_block
        bm = band_random_block_mask(nb)
        if w.name == "C5":
            assert int(bm.sum()) == C5_KEPT_BLOCKS, int(bm.sum())
    return {"q": q, "k": k, "v": v, "do": do, "block_mask": bm}
