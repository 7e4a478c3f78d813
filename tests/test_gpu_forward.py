"""GPU parity of the forward pass (O, LSE) against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

from tests._gpu import TOL, inputs, max_abs, note, oracle_fwd, to_dev
from workloads import random_block_mask

pytestmark = pytest.mark.gpu

DTYPES = [torch.bfloat16, torch.float16, torch.float32]


def _check_fwd(fa, B, H, N, d, dtype, causal=False, p=0.0, seed=0, bm=None, mb=128, k_scale=1.0, in_seed=7):
    note(f"fwd B={B} H={H} N={N} d={d} {dtype} causal={causal} p={p} block={bm is not None}")
    q, k, v, _ = inputs(B, H, N, d, dtype, in_seed, k_scale)
    scale = 1.0 / math.sqrt(d)
    qd, kd, vd = to_dev(q, k, v)
    o, lse = fa.forward(qd, kd, vd, scale=scale, causal=causal, dropout_p=p, seed=seed,
                        block_mask=None if bm is None else torch.from_numpy(bm), mask_block=mb)
    torch.cuda.synchronize()
    O, L = oracle_fwd(q, k, v, scale, causal, p, seed, bm, mb)
    eo = max_abs(o.float().cpu().numpy(), O)
    el = max_abs(lse.cpu().numpy(), L)
    tol = TOL[dtype]
    assert eo <= tol and el <= tol, (eo, el)
    return eo, el


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_small_shapes(fa, dtype, d, causal):
    for N in (1, 7, 64, 65, 129, 200):
        _check_fwd(fa, 1, 2, N, d, dtype, causal=causal, in_seed=N)


# A grid of 128-row tiles that would fill at most a quarter of the CUs
# (4 * tiles <= 256) takes a split-key kernel (32-row workgroups for 16-bit
# inputs, 16-row ones on 16x16x4 MFMAs for fp32; the keys dealt over four
# waves, partial results merged in LDS); the shapes above mostly take it.
# The same cases with 68 heads take the 128-row kernel.
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_small_shapes_wide_grid(fa, dtype, d, causal):
    for N in (1, 65, 200):
        _check_fwd(fa, 4, 17, N, d, dtype, causal=causal, in_seed=N + 3)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
def test_forward_dropout_and_block_mask_both_kernels(fa, dtype, d):
    N, mb = 1000, 128
    bm = random_block_mask((N + mb - 1) // mb, seed=d, frac=0.4)
    for B, H in ((1, 2), (4, 9)):  # 16 tiles (split-key kernel), 288 tiles (128-row kernel)
        _check_fwd(fa, B, H, N, d, dtype, causal=True, p=0.1, seed=0x5EED0003, bm=bm, mb=mb,
                   in_seed=B * H + d)


@pytest.mark.parametrize("N", [127, 128, 300, 1000])
def test_forward_tails_and_multiple_tiles(fa, N):
    _check_fwd(fa, 2, 2, N, 64, torch.bfloat16, causal=True, in_seed=N + 1)
    _check_fwd(fa, 1, 3, N, 128, torch.bfloat16, causal=False, in_seed=N + 2)


@pytest.mark.parametrize("B,H,N,d,dtype", [
    (1, 8, 4001, 64, torch.bfloat16),   # 32 tiles x 8 heads, 4 workgroups per CU, ragged tail
    (2, 8, 2000, 64, torch.float32),    # 16 tiles x 16 heads, 2 workgroups per CU
    (1, 8, 4001, 128, torch.float16),   # 32 tiles x 8 heads, 2 workgroups per CU
])
def test_forward_causal_grids_resident_at_once(fa, B, H, N, d, dtype):
    # causal grids that fit the chip in one round take the balanced
    # (serpentine) tile order; every head is checked whole
    _check_fwd(fa, B, H, N, d, dtype, causal=True, in_seed=N + d)


def test_forward_causal_grid_resident_at_once_with_dropout(fa):
    # dropout indexes by (b, h, query, key), whatever workgroup computes the tile
    _check_fwd(fa, 1, 8, 4001, 64, torch.bfloat16, causal=True, p=0.2, seed=77, in_seed=9)


def test_forward_workload_c1_fp32(fa):
    # single-head, non-causal, fp32, N=128, d=64 at its full size
    from workloads import WORKLOADS, workload_inputs

    w = WORKLOADS["C1"]
    x = workload_inputs(w)
    note("fwd workload C1")
    qd, kd, vd = to_dev(x["q"], x["k"], x["v"])
    o, lse = fa.forward(qd, kd, vd, scale=w.scale)
    torch.cuda.synchronize()
    O, L = oracle_fwd(x["q"], x["k"], x["v"], w.scale)
    assert max_abs(o.cpu().numpy(), O) <= 1e-4
    assert max_abs(lse.cpu().numpy(), L) <= 1e-4


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
def test_forward_dropout(fa, dtype, d):
    _check_fwd(fa, 2, 2, 300, d, dtype, causal=True, p=0.1, seed=0x5EED0003)
    _check_fwd(fa, 1, 2, 130, d, dtype, causal=False, p=0.5, seed=2**63 + 12345)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_block_sparse(fa, d, causal):
    N, mb = 1000, 128
    nb = (N + mb - 1) // mb
    bm = random_block_mask(nb, seed=d + causal, frac=0.3)
    _check_fwd(fa, 1, 2, N, d, torch.bfloat16, causal=causal, bm=bm, mb=mb)
    bm256 = random_block_mask((N + 255) // 256, seed=3, frac=0.5)
    _check_fwd(fa, 1, 2, N, d, torch.bfloat16, causal=causal, bm=bm256, mb=256)


def test_forward_fully_masked_rows(fa):
    # a block-mask row with no kept block: O = 0, LSE = -inf
    N, mb = 384, 128
    bm = np.array([[0, 0, 0], [1, 1, 0], [0, 1, 1]], dtype=np.uint8)
    _check_fwd(fa, 1, 1, N, 64, torch.bfloat16, bm=bm, mb=mb)
    q, k, v, _ = inputs(1, 1, N, 64, torch.bfloat16, 5)
    o, lse = fa.forward(*to_dev(q, k, v), block_mask=torch.from_numpy(bm), mask_block=mb)
    torch.cuda.synchronize()
    assert torch.all(o[0, 0, :128] == 0) and torch.all(torch.isneginf(lse[0, 0, :128]))


def test_forward_p_zero_equals_no_dropout_bitwise(fa):
    q, k, v, _ = inputs(1, 2, 200, 64, torch.bfloat16, 9)
    qd, kd, vd = to_dev(q, k, v)
    o1, l1 = fa.forward(qd, kd, vd, causal=True)
    o2, l2 = fa.forward(qd, kd, vd, causal=True, dropout_p=0.0, seed=1234)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_forward_deterministic(fa):
    q, k, v, _ = inputs(2, 4, 777, 128, torch.bfloat16, 10)
    qd, kd, vd = to_dev(q, k, v)
    o1, l1 = fa.forward(qd, kd, vd, causal=True, dropout_p=0.2, seed=5)
    o2, l2 = fa.forward(qd, kd, vd, causal=True, dropout_p=0.2, seed=5)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# The forward tile loop is unrolled by two (each step's LDS buffers fixed at
# compile time), so whether a workgroup's tile count is odd or even decides
# which copy ends the loop. Non-causal, 64-key tiles, a grid wide enough
# for the 128-row kernel: 1, 2, 3 and 5 tiles per workgroup.
@pytest.mark.parametrize("d", [64, 128])
def test_forward_tile_count_parity(fa, d):
    for N in (64, 128, 192, 320):
        _check_fwd(fa, 4, 17, N, d, torch.bfloat16, causal=False, in_seed=N + 5)
