"""GPU parity over a seeded random sample of option combinations, forward and
backward against the fp64 oracle at the fixed bounds (1e-4 fp32, 2e-2 for
16-bit inputs): batch and head counts, ragged lengths, head size, input
dtype, causal or not, block-sparse masks of either block size (with or
without their diagonal, so some rows see no key), dropout, the softmax scale,
the gradient precision, and grids on both sides of the small-grid switch.
The targeted tests spell out the edge cases one by one; this sample covers
pairings of options that they do not name. Inputs are N(0, 1) at scales of
at most 1/sqrt(d), the conditions the fixed bounds are stated for."""
import math

import numpy as np
import pytest
import torch

from tests._gpu import TOL, inputs, max_abs, note, oracle_bwd, oracle_fwd, to_dev
from workloads import random_block_mask

pytestmark = pytest.mark.gpu

DTYPES = (torch.bfloat16, torch.float16, torch.float32)


def _cases(n=40, seed=20261203):
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = DTYPES[int(r.integers(3))]
        d = int(r.choice([64, 128]))
        B = int(r.integers(1, 4))
        H = int(r.choice([1, 2, 3, 5, 17]))
        N = int(r.integers(1, 700)) if H < 17 else int(r.integers(1, 300))
        causal = bool(r.integers(2))
        p = float(r.choice([0.0, 0.0, 0.1, 0.2]))
        mb = int(r.choice([0, 128, 256]))  # 0: no block mask
        keep_diag = bool(r.integers(2))
        scale_mul = float(r.choice([1.0, 0.5]))  # times 1 / sqrt(d)
        grad = "input" if dtype == torch.float16 and r.integers(2) else "fp32"
        out.append((i, dtype, d, B, H, N, causal, p, mb, keep_diag, scale_mul, grad))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[f"case{c[0]}" for c in CASES])
def test_random_option_combination(fa, case):
    i, dtype, d, B, H, N, causal, p, mb, keep_diag, scale_mul, grad = case
    scale = scale_mul / math.sqrt(d)
    bm = None
    if mb:
        nb = (N + mb - 1) // mb
        bm = random_block_mask(nb, seed=1000 + i, frac=0.6, keep_diag=keep_diag)
    seed = 0xABC000 + i
    note(f"random case {i}: B={B} H={H} N={N} d={d} {dtype} causal={causal} p={p} mb={mb} "
         f"diag={keep_diag} scale={scale:.4f} grads={grad}")
    q, k, v, do = inputs(B, H, N, d, dtype, 5000 + i)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    kw = dict(scale=scale, causal=causal, dropout_p=p, seed=seed,
              block_mask=None if bm is None else torch.from_numpy(bm), mask_block=mb or 128)
    o, lse = fa.forward(qd, kd, vd, **kw)
    grad_dtype = dtype if grad == "input" else torch.float32
    dq, dk, dv = fa.backward(qd, kd, vd, o, lse, dod, grad_dtype=grad_dtype, **kw)
    torch.cuda.synchronize()
    O, L = oracle_fwd(q, k, v, scale, causal, p, seed, bm, mb or 128)
    G = oracle_bwd(q, k, v, do, scale, causal, p, seed, bm, mb or 128)
    errs = {"O": max_abs(o.float().cpu().numpy(), O), "LSE": max_abs(lse.cpu().numpy(), L)}
    for name, got, ref in zip(("dQ", "dK", "dV"), (dq, dk, dv), G):
        assert got.dtype == grad_dtype
        errs[name] = max_abs(got.float().cpu().numpy(), ref)
    assert all(e <= TOL[dtype] for e in errs.values()), errs
