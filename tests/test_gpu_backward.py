"""GPU parity of the backward pass (dQ, dK, dV) against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
from tests._gpu import TOL, inputs, max_abs, note, oracle_bwd, to_dev
from workloads import random_block_mask

pytestmark = pytest.mark.gpu


def _check_bwd(fa, B, H, N, d, dtype, causal=False, p=0.0, seed=0, bm=None, mb=128, in_seed=11,
               grad_dtype=torch.float32, tol=None):
    note(f"bwd B={B} H={H} N={N} d={d} {dtype} causal={causal} p={p} block={bm is not None} grad={grad_dtype}")
    q, k, v, do = inputs(B, H, N, d, dtype, in_seed)
    scale = 1.0 / math.sqrt(d)
    kw = dict(scale=scale, causal=causal, dropout_p=p, seed=seed,
              block_mask=None if bm is None else torch.from_numpy(bm), mask_block=mb)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    o, lse = fa.forward(qd, kd, vd, **kw)
    dq, dk, dv = fa.backward(qd, kd, vd, o, lse, dod, grad_dtype=grad_dtype, **kw)
    torch.cuda.synchronize()
    rq, rk, rv = oracle_bwd(q, k, v, do, scale, causal, p, seed, bm, mb)
    tol = TOL[dtype] if tol is None else tol
    errs = [max_abs(x.float().cpu().numpy(), r) for x, r in ((dq, rq), (dk, rk), (dv, rv))]
    assert max(errs) <= tol, errs
    return errs


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_small_shapes(fa, dtype, d, causal):
    for N in (1, 7, 64, 65, 129, 200):
        _check_bwd(fa, 1, 2, N, d, dtype, causal=causal, in_seed=N + 3)


@pytest.mark.parametrize("N", [255, 256, 640, 1000])
def test_backward_tails_and_multiple_tiles(fa, N):
    _check_bwd(fa, 2, 2, N, 64, torch.bfloat16, causal=True, in_seed=N)
    _check_bwd(fa, 1, 2, N, 128, torch.bfloat16, causal=False, in_seed=N + 1)
    # d = 128 causal: 256-key dK/dV workgroups whose diagonal rows leave
    # some waves idle, and a ragged last key block
    _check_bwd(fa, 1, 3, N, 128, torch.bfloat16, causal=True, in_seed=N + 2)


def test_backward_causal_sixteen_heads_ragged(fa):
    # 16 query tiles x 16 heads (ragged last tile): a causal grid that fits
    # the chip in one round; every head checked whole
    _check_bwd(fa, 1, 16, 2001, 64, torch.bfloat16, causal=True, in_seed=21)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
def test_backward_dropout(fa, dtype, d):
    _check_bwd(fa, 2, 2, 300, d, dtype, causal=True, p=0.1, seed=0x5EED0003)
    _check_bwd(fa, 1, 2, 130, d, dtype, causal=False, p=0.5, seed=2**63 + 99)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_block_sparse(fa, d, causal):
    N, mb = 1000, 128
    bm = random_block_mask((N + mb - 1) // mb, seed=10 + d + causal, frac=0.3)
    _check_bwd(fa, 1, 2, N, d, torch.bfloat16, causal=causal, bm=bm, mb=mb)
    bm256 = random_block_mask((N + 255) // 256, seed=4, frac=0.5)
    _check_bwd(fa, 1, 2, N, d, torch.bfloat16, causal=causal, bm=bm256, mb=256)


def test_backward_fully_masked_rows_have_zero_gradient(fa):
    N, mb = 384, 128
    bm = np.array([[0, 0, 0], [1, 1, 0], [0, 1, 1]], dtype=np.uint8)
    _check_bwd(fa, 1, 2, N, 64, torch.bfloat16, bm=bm, mb=mb)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_backward_low_precision_gradients(fa, dtype):
    # gradients written in the input dtype: compare with the fp32-gradient
    # result (same kernels) within one rounding of the output, and with the
    # oracle within the input-dtype tolerance
    q, k, v, do = inputs(1, 2, 333, 64, dtype, 21)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    o, lse = fa.forward(qd, kd, vd, causal=True)
    g32 = fa.backward(qd, kd, vd, o, lse, dod, causal=True)
    g16 = fa.backward(qd, kd, vd, o, lse, dod, causal=True, grad_dtype=dtype)
    torch.cuda.synchronize()
    for a, b in zip(g32, g16):
        assert b.dtype == dtype
        assert torch.equal(a.to(dtype), b)
    _check_bwd(fa, 1, 2, 333, 64, dtype, causal=True, in_seed=21, grad_dtype=dtype)


def test_backward_deterministic(fa):
    q, k, v, do = inputs(2, 3, 517, 128, torch.bfloat16, 31)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    o, lse = fa.forward(qd, kd, vd, causal=True, dropout_p=0.2, seed=7)
    g1 = fa.backward(qd, kd, vd, o, lse, dod, causal=True, dropout_p=0.2, seed=7)
    g2 = fa.backward(qd, kd, vd, o, lse, dod, causal=True, dropout_p=0.2, seed=7)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("p", [0.1, 0.3])
def test_keep_bits_used_inside_backward(fa, p):
    # Q = 0 makes P uniform (1/128) over one kept 128-key block per row
    # block; the kept column blocks form a permutation so every key block is
    # seen by exactly one query block.
    #  dK/dV kernel: dO_i = e_{i mod 128} gives dV_j[i mod 128] = Z_ij / (128 (1 - p)).
    #  dQ kernel:    K_j = e_{j mod 128}, V_j = 1, dO_i = e_0 give
    #                dQ_i[j mod 128] = scale/128 * (Z_ij / (1 - p) - D_i).
    N, d, mb = 512, 128, 128
    nb = N // mb
    perm = np.random.default_rng(2).permutation(nb)
    bm = np.zeros((nb, nb), np.uint8)
    bm[np.arange(nb), perm] = 1
    B, H, seed, dtype = 1, 2, 0xFEEDFACE, torch.bfloat16
    scale = 1.0 / math.sqrt(d)
    ar = torch.arange(N)
    q = torch.zeros(B, H, N, d, dtype=dtype)
    kk = torch.zeros(B, H, N, d, dtype=dtype)
    kk[:, :, ar, ar % 128] = 1
    v_ones = torch.ones(B, H, N, d, dtype=dtype)
    do_onehot = torch.zeros(B, H, N, d, dtype=dtype)
    do_onehot[:, :, ar, ar % 128] = 1
    do_e0 = torch.zeros(B, H, N, d, dtype=dtype)
    do_e0[:, :, :, 0] = 1
    kw = dict(scale=scale, dropout_p=p, seed=seed, block_mask=torch.from_numpy(bm), mask_block=mb)
    note(f"dropout probe bwd p={p}")
    qd, kd, vd = to_dev(q, kk, v_ones)
    o, lse = fa.forward(qd, kd, vd, **kw)
    _, _, dv = fa.backward(qd, kd, vd, o, lse, do_onehot.cuda(), **kw)
    dq, _, _ = fa.backward(qd, kd, vd, o, lse, do_e0.cuda(), **kw)
    torch.cuda.synchronize()
    dv = dv.cpu().numpy()
    dq = dq.cpu().numpy()
    for b in range(B):
        for h in range(H):
            for r in range(nb):
                rows = np.arange(r * mb, (r + 1) * mb)
                keys = np.arange(perm[r] * mb, (perm[r] + 1) * mb)
                Z = oracle.dropout_keep(seed, b, h, rows, keys, p)
                # dV_j[i mod 128] for j in the block, i in the row block
                got = dv[b, h][keys][:, rows % 128].T * 128 * (1 - p)
                np.testing.assert_array_equal(np.rint(got).astype(bool), Z)
                assert np.abs(got - np.rint(got)).max() < 0.05
                # dQ_i[j mod 128] = scale/128 * (Z_ij/(1-p) - D_i)
                g = dq[b, h][rows][:, keys % 128] * 128 / scale
                lvl = (g - g.min(axis=1, keepdims=True)) * (1 - p)
                np.testing.assert_array_equal(np.rint(lvl).astype(bool), Z)
                assert np.abs(lvl - np.rint(lvl)).max() < 0.05


@pytest.mark.parametrize("N", [2100, 4500])
@pytest.mark.parametrize("causal,p", [(True, 0.0), (False, 0.0), (True, 0.1)])
def test_backward_long_rows(fa, N, causal, p):
    # longer sequences take the large-tile launch configurations (with tails)
    _check_bwd(fa, 1, 1, N, 64, torch.bfloat16, causal=causal, p=p, seed=0x5EED0003, in_seed=N + 5)


def test_side_stream_gives_identical_results(fa):
    # every call enqueues on the caller's current stream; the library keeps
    # no state, so a side stream yields the same bits as the default stream
    q, k, v, do = inputs(2, 3, 300, 64, torch.bfloat16, 41)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    kw = dict(causal=True, dropout_p=0.1, seed=11)
    note("side stream fwd+bwd")
    o1, l1 = fa.forward(qd, kd, vd, **kw)
    g1 = fa.backward(qd, kd, vd, o1, l1, dod, **kw)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o2, l2 = fa.forward(qd, kd, vd, **kw)
        g2 = fa.backward(qd, kd, vd, o2, l2, dod, **kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for a, b in zip((o1, l1) + tuple(g1), (o2, l2) + tuple(g2)):
        assert torch.equal(a, b)


def test_block_mask_wider_than_64_blocks(fa):
    # masks of up to 64 blocks per row are read once into a 64-bit word;
    # wider ones (here 66 blocks of 128) are walked byte by byte
    N, mb = 8400, 128
    bm = random_block_mask((N + mb - 1) // mb, seed=66, frac=0.1)
    _check_bwd(fa, 1, 1, N, 64, torch.bfloat16, causal=False, bm=bm, mb=mb, in_seed=8400)


# The same for the backward loops (unrolled by two in the dQ kernel, and in
# the dK/dV kernel at d = 64 with 32-row query tiles): 1, 3, 5 and 6 tiles
# of 32 rows or keys, and 1 to 3 of 64.
@pytest.mark.parametrize("d", [64, 128])
def test_backward_tile_count_parity(fa, d):
    for N in (32, 96, 160, 192):
        _check_bwd(fa, 2, 4, N, d, torch.bfloat16, causal=False, in_seed=N + 6)
