"""Parity at long sequence lengths (16K to 64K tokens per head), where the
oracle cannot form a whole N x N head: query rows are checked one by one
(O, LSE, dQ), keys from their whole rows' statistics (dK, dV), plus
properties that hold at any N (sum_j dK_j = 0; sum_j dV_j = sum_i dO_i
without dropout, since each row of P sums to one)."""
import math

import numpy as np
import pytest
import torch

import oracle
from tests._gpu import TOL, max_abs, note
from workloads import DROPOUT_SEED, draw_qkvdo

pytestmark = pytest.mark.gpu

# (N, d, causal, dropout_p); causal heads are checked on their last keys,
# which few rows see, the non-causal one on keys spread over the sequence
CASES = [
    (65536, 64, True, 0.0),
    (32768, 128, True, 0.0),
    (32768, 64, True, 0.1),
    (16384, 64, False, 0.0),
]


@pytest.mark.parametrize("N,d,causal,p", CASES, ids=[f"N{c[0]}-d{c[1]}-{'causal' if c[2] else 'dense'}-p{c[3]}"
                                                     for c in CASES])
def test_long_sequence(fa, N, d, causal, p):
    B, H = 1, 2
    scale = 1.0 / math.sqrt(d)
    seed = DROPOUT_SEED if p > 0 else 0
    note(f"long sequence B={B} H={H} N={N} d={d} causal={causal} p={p}")
    q, k, v, do = draw_qkvdo(B, H, N, d, torch.bfloat16, 7000 + N + d)
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    kw = dict(scale=scale, causal=causal, dropout_p=p, seed=seed)
    o, lse = fa.forward(qd, kd, vd, **kw)
    dq, dk, dv = fa.backward(qd, kd, vd, o, lse, dod, **kw)
    torch.cuda.synchronize()
    o, lse, dq, dk, dv = (t.float().cpu().numpy() for t in (o, lse, dq, dk, dv))
    tol = TOL[torch.bfloat16]
    rng = np.random.default_rng(N + d)
    rows = np.unique(np.concatenate([[0, 1, N // 2, N - 1], rng.integers(0, N, 12)]))
    if causal:
        cols = np.unique(np.concatenate([[N - 1, N - 64, N - 65], rng.integers(N - 400, N, 9)]))
    else:
        cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 6)]))
    for h in range(H):
        O, L = oracle.forward_rows(q, k, v, scale, 0, h, rows, causal, p, seed)
        G = oracle.backward_rows(q, k, v, do, scale, 0, h, rows, causal, p, seed)
        gk, gv = oracle.backward_cols(q, k, v, do, scale, 0, h, cols, causal, p, seed)
        errs = {"O": max_abs(o[0, h][rows], O), "LSE": max_abs(lse[0, h][rows], L),
                "dQ": max_abs(dq[0, h][rows], G), "dK": max_abs(dk[0, h][cols], gk),
                "dV": max_abs(dv[0, h][cols], gv)}
        assert max(errs.values()) <= tol, (h, errs)
        assert np.isfinite(o[0, h]).all() and np.isfinite(dq[0, h]).all()
        assert np.isfinite(dk[0, h]).all() and np.isfinite(dv[0, h]).all()
        # properties over every key: sum_j dK_j = 0 always; sum_j dV_j = sum_i dO_i
        # without dropout. Per-element errors are ~1e-3 and largely independent,
        # so the bound grows like sqrt(N).
        bound = 2e-2 * math.sqrt(N)
        assert np.abs(dk[0, h].astype(np.float64).sum(axis=0)).max() < bound
        if p == 0:
            ref = do[0, h].double().sum(dim=0).numpy()
            assert np.abs(dv[0, h].astype(np.float64).sum(axis=0) - ref).max() < bound
