"""Pins of the oracle's backward pass (dQ, dK, dV) against things other than itself.

CPU only. Central finite differences of L = sum(O * dO) on the oracle's
forward (which is itself pinned), torch autograd in float64 on the explicit
formula, and identities (D_i = dO_i . O_i, sum_j dK_j = 0, closed form at
Q = 0, permutation equivariance).
"""
import math

import numpy as np
import pytest
import torch

import oracle

MODES = [(False, False), (True, False), (False, True), (True, True)]


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _bm(nb, seed):
    m = (np.random.default_rng(seed).random((nb, nb)) < 0.6).astype(np.uint8)
    m[np.arange(nb), np.arange(nb)] = 1
    return m


def _loss(q, k, v, do, kw):
    O, _ = oracle.forward_head(q, k, v, **kw)
    return float((O * do).sum())


@pytest.mark.parametrize("causal,block", MODES)
@pytest.mark.parametrize("p", [0.0, 0.3])
def test_backward_matches_central_finite_differences(causal, block, p):
    N, d, mb = 11, 3, 4
    q, k, v, do = (_rand((N, d), s) for s in (1, 2, 3, 4))
    kw = dict(scale=0.8, causal=causal, dropout_p=p, seed=1234, b=1, h=0,
              block_mask=_bm(3, 5) if block else None, mask_block=mb)
    g = oracle.backward_head(q, k, v, do, **kw)
    eps = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"dq": (xp, k, v), "dk": (q, xp, v), "dv": (q, k, xp)}[name]
            args_m = {"dq": (xm, k, v), "dk": (q, xm, v), "dv": (q, k, xm)}[name]
            fd[idx] = (_loss(*args_p, do, kw) - _loss(*args_m, do, kw)) / (2 * eps)
        err = np.abs(fd - g[name]).max() / max(1.0, np.abs(fd).max())
        assert err < 1e-6, (name, err)


@pytest.mark.parametrize("causal,block", MODES)
@pytest.mark.parametrize("p", [0.0, 0.2])
def test_backward_matches_torch_autograd_float64(causal, block, p):
    N, d, mb = 37, 8, 8
    q, k, v, do = (_rand((N, d), s) for s in (11, 12, 13, 14))
    bm = _bm(5, 15) if block else None
    scale, seed, b, h = 0.35, 99, 0, 3
    g = oracle.backward_head(q, k, v, do, scale, causal, p, seed, b, h, bm, mb)
    valid = torch.from_numpy(oracle.valid_mask(N, causal, bm, mb))
    Z = torch.from_numpy(oracle.dropout_keep(seed, b, h, np.arange(N), np.arange(N), p)).double()
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    s = scale * tq @ tk.T
    s = s.masked_fill(~valid, -math.inf)
    P = torch.softmax(s, dim=1)
    O = (P * Z / (1 - p)) @ tv
    O.backward(torch.from_numpy(do))
    np.testing.assert_allclose(g["dq"], tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(g["dk"], tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(g["dv"], tv.grad.numpy(), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.0, 0.15])
def test_identities(causal, p):
    N, d = 64, 16
    q, k, v, do = (_rand((N, d), s) for s in (21, 22, 23, 24))
    kw = dict(causal=causal, dropout_p=p, seed=4321, b=2, h=5)
    g = oracle.backward_head(q, k, v, do, 0.25, **kw)
    O, _ = oracle.forward_head(q, k, v, 0.25, **kw)
    # D_i = sum_j P_ij dP_ij equals dO_i . O_i
    np.testing.assert_allclose(g["D"], (do * O).sum(axis=1), atol=1e-12)
    # softmax is invariant to adding a constant to a row, so sum_j dS_ij = 0
    # and hence sum_j dK_j = 0
    np.testing.assert_allclose(g["dk"].sum(axis=0), 0.0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.0, 0.3])
def test_closed_form_zero_queries(causal, p):
    # Q = 0: dK = 0 (dK is a combination of Q rows) and
    # dV_j = sum over rows i that see j of Z_ij dO_i / (n_i (1 - p))
    N, d = 21, 3
    q = np.zeros((N, d))
    k, v, do = (_rand((N, d), s) for s in (31, 32, 33))
    g = oracle.backward_head(q, k, v, do, 0.5, causal, p, 8, 0, 0)
    np.testing.assert_array_equal(g["dk"], 0.0)
    Z = oracle.dropout_keep(8, 0, 0, np.arange(N), np.arange(N), p)
    n = np.arange(1, N + 1) if causal else np.full(N, N)
    for j in range(N):
        rows = np.arange(j, N) if causal else np.arange(N)
        expect = (Z[rows, j, None] * do[rows] / (n[rows, None] * (1 - p))).sum(axis=0)
        np.testing.assert_allclose(g["dv"][j], expect, atol=1e-13)


def test_permutation_equivariance_of_dk_dv():
    N, d = 29, 4
    q, k, v, do = (_rand((N, d), s) for s in (41, 42, 43, 44))
    perm = np.random.default_rng(45).permutation(N)
    g1 = oracle.backward_head(q, k, v, do, 0.5)
    g2 = oracle.backward_head(q, k[perm], v[perm], do, 0.5)
    np.testing.assert_allclose(g2["dk"], g1["dk"][perm], atol=1e-13)
    np.testing.assert_allclose(g2["dv"], g1["dv"][perm], atol=1e-13)
    np.testing.assert_allclose(g2["dq"], g1["dq"], atol=1e-13)


def test_batched_backward_matches_heads():
    B, H, N, d = 2, 2, 10, 4
    rng = np.random.default_rng(51)
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    dq, dk, dv = oracle.backward(q, k, v, do, 0.5, causal=True, dropout_p=0.1, seed=3)
    g = oracle.backward_head(q[1, 0], k[1, 0], v[1, 0], do[1, 0], 0.5, True, 0.1, 3, 1, 0)
    np.testing.assert_array_equal(dq[1, 0], g["dq"])
    np.testing.assert_array_equal(dk[1, 0], g["dk"])
    np.testing.assert_array_equal(dv[1, 0], g["dv"])


@pytest.mark.parametrize("causal,p", [(False, 0.0), (True, 0.0), (True, 0.25)])
def test_backward_rows_matches_finite_differences(causal, p):
    # dQ of a few rows from their own definition, against central differences
    # of L = sum(O * dO) with respect to those rows of Q
    B, H, N, d = 1, 2, 13, 3
    rng = np.random.default_rng(61)
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    rows = [0, 5, 12]
    kw = dict(causal=causal, dropout_p=p, seed=17)
    g = oracle.backward_rows(q, k, v, do, 0.6, 0, 1, rows, **kw)
    eps = 1e-6
    for a, i in enumerate(rows):
        for c in range(d):
            qp, qm = q.copy(), q.copy()
            qp[0, 1, i, c] += eps
            qm[0, 1, i, c] -= eps
            lp = (oracle.forward_head(qp[0, 1], k[0, 1], v[0, 1], 0.6, b=0, h=1, **kw)[0] * do[0, 1]).sum()
            lm = (oracle.forward_head(qm[0, 1], k[0, 1], v[0, 1], 0.6, b=0, h=1, **kw)[0] * do[0, 1]).sum()
            assert abs((lp - lm) / (2 * eps) - g[a, c]) < 1e-6
    full = oracle.backward_head(q[0, 1], k[0, 1], v[0, 1], do[0, 1], 0.6, b=0, h=1, **kw)["dq"]
    np.testing.assert_allclose(g, full[rows], atol=1e-12)


@pytest.mark.parametrize("causal,block,p", [(False, False, 0.0), (True, False, 0.0), (True, True, 0.25),
                                            (False, True, 0.1)])
def test_backward_cols_matches_finite_differences(causal, block, p):
    # dK, dV of a few keys, against central differences of L = sum(O * dO)
    # with respect to those rows of K and V (row_chunk=4 spans several chunks)
    B, H, N, d, mb = 2, 1, 13, 3, 4
    rng = np.random.default_rng(71)
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    bm = _bm(4, 72) if block else None
    cols = [0, 6, 12]
    kw = dict(causal=causal, dropout_p=p, seed=23, block_mask=bm, mask_block=mb)
    gk, gv = oracle.backward_cols(q, k, v, do, 0.7, 1, 0, cols, row_chunk=4, **kw)

    def loss(kk, vv):
        return (oracle.forward_head(q[1, 0], kk, vv, 0.7, b=1, h=0, **kw)[0] * do[1, 0]).sum()

    eps = 1e-6
    for a, j in enumerate(cols):
        for c in range(d):
            for g, which in ((gk, 0), (gv, 1)):
                xp = [k[1, 0].copy(), v[1, 0].copy()]
                xm = [k[1, 0].copy(), v[1, 0].copy()]
                xp[which][j, c] += eps
                xm[which][j, c] -= eps
                assert abs((loss(*xp) - loss(*xm)) / (2 * eps) - g[a, c]) < 1e-6
    full = oracle.backward_head(q[1, 0], k[1, 0], v[1, 0], do[1, 0], 0.7, b=1, h=0, **kw)
    np.testing.assert_allclose(gk, full["dk"][cols], atol=1e-12)
    np.testing.assert_allclose(gv, full["dv"][cols], atol=1e-12)
