"""Dropout keep bits: the device hash must match the oracle bit for bit,
both through fa_dropout_mask and as actually used inside the fused kernels."""
import math

import numpy as np
import pytest
import torch

import oracle
from tests._gpu import note, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9, 1e-9])
def test_dropout_mask_bit_exact(fa, p):
    seeds = [0, 0x5EED0003, 2**64 - 1, 0x0123456789ABCDEF]
    B, H, N = 4, 16, 16400
    for seed in seeds:
        for (b, h, i0, rows, j0, cols) in [(0, 0, 0, 64, 0, 257), (3, 15, 16300, 100, 16000, 400),
                                           (1, 7, 8191, 3, 0, 16400)]:
            note(f"dropout_mask p={p} seed={seed:#x} b={b} h={h} i0={i0} j0={j0}")
            keep = fa.dropout_mask(B, H, N, 64, b, h, i0, rows, j0, cols, dropout_p=p, seed=seed)
            torch.cuda.synchronize()
            ref = oracle.dropout_keep(seed, b, h, np.arange(i0, i0 + rows), np.arange(j0, j0 + cols), p)
            np.testing.assert_array_equal(keep.cpu().numpy().astype(bool), ref)


def test_dropout_mask_p_zero_all_kept(fa):
    keep = fa.dropout_mask(1, 1, 300, 64, 0, 0, 0, 300, 0, 300, dropout_p=0.0, seed=9)
    torch.cuda.synchronize()
    assert bool(keep.all())


@pytest.mark.parametrize("p", [0.1, 0.3])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_keep_bits_used_inside_forward(fa, p, dtype):
    # Probe: Q = 0 makes P uniform (1/128) over one kept 128-key block per
    # row block; V rows are one-hot (V_j = e_{j mod 128}), so
    # O_{i, j mod 128} = Z_ij / (128 (1 - p)) decodes every keep bit the
    # fused forward used for the kept block.
    N, d, mb = 512, 128, 128
    nb = N // mb
    rng = np.random.default_rng(1)
    cols = rng.integers(0, nb, size=nb)
    bm = np.zeros((nb, nb), np.uint8)
    bm[np.arange(nb), cols] = 1
    B, H, seed = 2, 3, 0xDEADBEEF12345
    q = torch.zeros(B, H, N, d, dtype=dtype)
    k = torch.randn(B, H, N, d).to(dtype)
    v = torch.zeros(B, H, N, d, dtype=dtype)
    v[:, :, torch.arange(N), torch.arange(N) % 128] = 1
    note(f"dropout probe fwd p={p} {dtype}")
    o, lse = fa.forward(*to_dev(q, k, v), dropout_p=p, seed=seed, block_mask=torch.from_numpy(bm), mask_block=mb)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    unit = 1.0 / (128 * (1 - p))
    for b in range(B):
        for h in range(H):
            for r in range(nb):
                rows = np.arange(r * mb, (r + 1) * mb)
                keys = np.arange(cols[r] * mb, (cols[r] + 1) * mb)
                Z = oracle.dropout_keep(seed, b, h, rows, keys, p)
                got = o[b, h, rows][:, keys % 128] / unit
                np.testing.assert_array_equal(np.rint(got).astype(bool), Z)
                assert np.abs(got - np.rint(got)).max() < 0.02
            np.testing.assert_allclose(lse.cpu().numpy()[b, h], math.log(128), atol=1e-5)


@pytest.mark.parametrize("N", [1024, 4096, 4608])
@pytest.mark.parametrize("p", [0.1, 0.37])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_keep_bits_inside_d64_kernels(fa, N, p, dtype):
    # The d = 64 launch configurations (the dropout workload's: forward with
    # 64-key tiles, dQ with 32-key tiles up to 4096 keys and 64-key tiles
    # beyond, dK/dV with 32-row tiles up to 2048 keys and 64-row tiles beyond)
    # decode every keep bit they use. Q = 0 and a permutation block mask make
    # P = 1/128 over one kept 128-key block per query block. Two-level one-hot
    # rows carry two bits per column: X_j = e_{j mod 64} * (1 if j mod 128 < 64
    # else 2), so a column of the product reads Z_1 + 2 Z_2 for the two keys
    # (or queries) that share it.
    #   forward, V = X:       O_i[c]  = (Z_{i,j0+c} + 2 Z_{i,j0+64+c}) / (128 (1 - p))
    #   dK/dV,   dO = X:      dV_j[c] = (Z_{i0+c,j} + 2 Z_{i0+64+c,j}) / (128 (1 - p))
    #   dQ, K = X, V = 1, dO = e_0:  D_i = O_i[0] and
    #                         dQ_i[c] = scale/128 * ((Z_{i,j0+c} + 2 Z_{i,j0+64+c}) / (1 - p) - 3 D_i)
    d, mb = 64, 128
    nb = N // mb
    perm = np.random.default_rng(N).permutation(nb)
    bm = np.zeros((nb, nb), np.uint8)
    bm[np.arange(nb), perm] = 1
    B, H, seed = 1, 2, 0xA5A5F00D0123
    scale = 1.0 / math.sqrt(d)
    ar = torch.arange(N)
    lvl = torch.where(ar % 128 < 64, 1.0, 2.0)
    X = torch.zeros(B, H, N, d)
    X[:, :, ar, ar % 64] = lvl
    X = X.to(dtype)
    q = torch.zeros(B, H, N, d, dtype=dtype)
    e0 = torch.zeros(B, H, N, d, dtype=dtype)
    e0[:, :, :, 0] = 1
    ones = torch.ones(B, H, N, d, dtype=dtype)
    kw = dict(scale=scale, dropout_p=p, seed=seed, block_mask=torch.from_numpy(bm), mask_block=mb)
    note(f"dropout probe d=64 N={N} p={p} {dtype}")
    krand = torch.randn(B, H, N, d).to(dtype)
    # forward and dK/dV: K arbitrary (Q = 0 ignores it), V = X, dO = X
    qd, kd, vd = to_dev(q, krand, X)
    o1, l1 = fa.forward(qd, kd, vd, **kw)
    _, _, dv = fa.backward(qd, kd, vd, o1, l1, X.cuda(), **kw)
    # dQ: K = X, V = 1, dO = e_0
    qd2, kd2, vd2 = to_dev(q, X, ones)
    o2, l2 = fa.forward(qd2, kd2, vd2, **kw)
    dq, _, _ = fa.backward(qd2, kd2, vd2, o2, l2, e0.cuda(), **kw)
    torch.cuda.synchronize()
    o1, dv, o2, dq = (t.float().cpu().numpy() for t in (o1, dv, o2, dq))
    u = 1.0 / (128 * (1 - p))

    def levels(x):
        r = np.rint(x)
        assert np.abs(x - r).max() < 0.1, np.abs(x - r).max()
        assert r.min() >= 0 and r.max() <= 3
        return r.astype(np.int64)

    for b in range(B):
        for h in range(H):
            for r in range(nb):
                rows = np.arange(r * mb, (r + 1) * mb)
                keys = np.arange(perm[r] * mb, (perm[r] + 1) * mb)
                Z = oracle.dropout_keep(seed, b, h, rows, keys, p).astype(np.int64)
                want_rows = Z[:, :64] + 2 * Z[:, 64:]      # [query][c]
                want_keys = Z[:64, :].T + 2 * Z[64:, :].T  # [key][c]
                np.testing.assert_array_equal(levels(o1[b, h][rows] / u), want_rows)
                np.testing.assert_array_equal(levels(dv[b, h][keys] / u), want_keys)
                D = o2[b, h][rows][:, :1]
                g = dq[b, h][rows] * 128 / scale
                np.testing.assert_array_equal(levels((g + 3 * D) * (1 - p)), want_rows)
