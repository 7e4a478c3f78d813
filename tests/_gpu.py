"""Helpers shared by the GPU parity tests: run the HIP path through the C
ABI binding and compare with the oracle element by element."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from workloads import draw_qkvdo

# Max-abs tolerances against the fp64 oracle, by input dtype.
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2, torch.float16: 2e-2}


def note(msg: str):
    """Name the case on stdout before a GPU step, flushed."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def max_abs(a, b, mask=None) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        d = np.where(both_inf, 0.0, np.abs(a - b))
    if mask is not None:
        d = d[mask]
    if d.size == 0:
        return 0.0
    return float(np.nanmax(np.where(np.isnan(d), np.inf, d)))


def inputs(B, H, N, d, dtype, seed, k_scale=1.0):
    return draw_qkvdo(B, H, N, d, dtype, seed, k_scale)


def to_dev(*ts):
    return [t.cuda() if t is not None else None for t in ts]


def oracle_fwd(q, k, v, scale, causal=False, dropout_p=0.0, seed=0, block_mask=None, mask_block=128, heads=None):
    return oracle.forward(q, k, v, scale, causal, dropout_p, seed, block_mask, mask_block, heads)


def oracle_bwd(q, k, v, do, scale, causal=False, dropout_p=0.0, seed=0, block_mask=None, mask_block=128,
               heads=None):
    return oracle.backward(q, k, v, do, scale, causal, dropout_p, seed, block_mask, mask_block, heads)
