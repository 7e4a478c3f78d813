"""CPU checks of the 16-bit textbook reference used to calibrate tolerances:
run in fp32 it is the plain algorithm and agrees with the fp64 oracle; in
bf16 its error is of the order of bf16 rounding."""
import numpy as np
import torch

from tests._gpu import inputs, max_abs, oracle_bwd, oracle_fwd
from tests._lowp_ref import lowp_attention
from workloads import random_block_mask


def test_fp32_reference_matches_oracle():
    B, H, N, d, mb, p, scale, seed = 2, 2, 150, 16, 32, 0.2, 0.4, 77
    bm = random_block_mask((N + mb - 1) // mb, seed=3, frac=0.6, keep_diag=False)
    q, k, v, do = inputs(B, H, N, d, torch.float32, 5)
    ref = lowp_attention(q, k, v, do, scale, True, p, seed, bm, mb)
    O, _ = oracle_fwd(q, k, v, scale, True, p, seed, bm, mb)
    G = oracle_bwd(q, k, v, do, scale, True, p, seed, bm, mb)
    for r, o in zip(ref, (O,) + tuple(G)):
        assert max_abs(r, o) < 1e-4


def test_bf16_reference_error_is_rounding_sized():
    B, H, N, d = 1, 2, 200, 32
    q, k, v, do = inputs(B, H, N, d, torch.bfloat16, 6)
    ref = lowp_attention(q, k, v, do, 1 / np.sqrt(d), True)
    O, _ = oracle_fwd(q, k, v, 1 / np.sqrt(d), True)
    G = oracle_bwd(q, k, v, do, 1 / np.sqrt(d), True)
    for r, o in zip(ref, (O,) + tuple(G)):
        e = max_abs(r, o)
        assert 1e-5 < e < 5e-2 * max(1.0, np.abs(o).max())
