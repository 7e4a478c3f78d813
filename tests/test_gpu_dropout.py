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
