"""Pins of the oracle's forward pass (O and LSE) against things other than itself.

CPU only. Each check targets a class of plausible mistakes:
* brute force at 50 digits (every mask mode, dropout): wrong scale, sign,
  transposed operand, mask index or dropout scaling;
* torch scaled_dot_product_attention in float64 (library special case);
* closed forms (Q = 0, N = 1, causal row 0, identical V rows);
* invariants (row sums, shift of K, joint permutation of K/V, permutation of
  Q, block masks that reduce to dense or causal, linearity in V).
"""
import math

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
from tests._brute import brute_forward

MODES = [
    dict(causal=False, block=False),
    dict(causal=True, block=False),
    dict(causal=False, block=True),
    dict(causal=True, block=True),
]


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _block_mask(nb, seed):
    m = (np.random.default_rng(seed).random((nb, nb)) < 0.5).astype(np.uint8)
    m[0, :] = 0  # row block 0 fully masked unless causal diagonal re-added below
    m[0, 0] = 1
    m[1 % nb, 0] = 0  # asymmetric pattern: (1,0) hidden, ...
    if nb > 1:
        m[0, 1] = 1  # ... (0,1) kept
    return m


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("p", [0.0, 0.3])
def test_forward_matches_brute_force_50_digits(mode, p):
    N, d, M, mb = 7, 3, 5, 2
    q, k, v = _rand((N, d), 1), _rand((N, d), 2), _rand((N, M), 3)
    v = v[:, :M]
    scale = 0.7
    bm = _block_mask((N + mb - 1) // mb, 4) if mode["block"] else None
    seed, b, h = 0xABCDEF0123, 2, 1
    O, L = oracle.forward_head(q, k, v, scale, causal=mode["causal"], dropout_p=p, seed=seed, b=b, h=h,
                               block_mask=bm, mask_block=mb)
    Ob, Lb = brute_forward(q.tolist(), k.tolist(), v.tolist(), scale, mode["causal"], bm, mb, p, seed, b, h)
    for i in range(N):
        if Lb[i] == -math.inf:
            assert L[i] == -np.inf
            assert np.all(O[i] == 0.0)
            continue
        assert abs(float(Lb[i]) - L[i]) < 1e-13
        for c in range(v.shape[1]):
            assert abs(float(Ob[i][c]) - O[i, c]) < 1e-13


def test_fully_masked_row_gives_zero_and_minus_inf():
    N, mb = 4, 2
    bm = np.array([[0, 0], [1, 1]], dtype=np.uint8)
    q, k, v = _rand((N, 3), 5), _rand((N, 3), 6), _rand((N, 3), 7)
    O, L = oracle.forward_head(q, k, v, 0.5, block_mask=bm, mask_block=mb)
    assert np.all(O[:2] == 0) and np.all(np.isneginf(L[:2]))
    assert np.all(np.isfinite(L[2:]))


def _sdpa_ref(q, k, v, scale, valid):
    tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (q, k, v))
    mask = torch.from_numpy(valid)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
    s = scale * (torch.from_numpy(q) @ torch.from_numpy(k).T)
    s = s.masked_fill(~torch.from_numpy(valid), -math.inf)
    return o[0, 0].numpy(), torch.logsumexp(s, dim=1).numpy()


@settings(max_examples=40, deadline=None)
@given(N=st.integers(1, 40), d=st.sampled_from([1, 2, 5, 8, 16]), causal=st.booleans(),
       block=st.booleans(), mb=st.sampled_from([1, 3, 8]), seed=st.integers(0, 10**6))
def test_forward_matches_torch_sdpa_float64(N, d, causal, block, mb, seed):
    q, k, v = _rand((N, d), seed), _rand((N, d), seed + 1), _rand((N, d), seed + 2)
    scale = 1.0 / math.sqrt(d)
    nb = (N + mb - 1) // mb
    bm = None
    if block:
        bm = (np.random.default_rng(seed + 3).random((nb, nb)) < 0.6).astype(np.uint8)
        bm[np.arange(nb), np.arange(nb)] = 1  # every row keeps its diagonal block
    valid = oracle.valid_mask(N, causal, bm, mb)
    O, L = oracle.forward_head(q, k, v, scale, causal=causal, block_mask=bm, mask_block=mb)
    Or, Lr = _sdpa_ref(q, k, v, scale, valid)
    np.testing.assert_allclose(O, Or, atol=1e-12, rtol=1e-12)
    np.testing.assert_allclose(L, Lr, atol=1e-12, rtol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.0, 0.25])
def test_closed_form_zero_queries(causal, p):
    # Q = 0 makes every visible score 0: P_ij = 1/n_i, LSE_i = ln n_i,
    # O_i = sum over visible j of Z_ij V_j / (n_i (1 - p))
    N, d = 33, 4
    q = np.zeros((N, d))
    k, v = _rand((N, d), 11), _rand((N, d), 12)
    O, L = oracle.forward_head(q, k, v, 0.3, causal=causal, dropout_p=p, seed=77, b=1, h=2)
    n = np.arange(1, N + 1) if causal else np.full(N, N)
    np.testing.assert_allclose(L, np.log(n), rtol=0, atol=1e-14)
    Z = oracle.dropout_keep(77, 1, 2, np.arange(N), np.arange(N), p)
    for i in range(N):
        vis = np.arange(n[i]) if causal else np.arange(N)
        expect = (Z[i, vis, None] * v[vis]).sum(axis=0) / (n[i] * (1 - p))
        np.testing.assert_allclose(O[i], expect, atol=1e-13)


def test_closed_form_single_token_and_causal_first_row():
    q, k, v = _rand((1, 6), 21), _rand((1, 6), 22), _rand((1, 6), 23)
    O, L = oracle.forward_head(q, k, v, 0.4)
    np.testing.assert_array_equal(O, v)
    assert abs(L[0] - 0.4 * float(q[0] @ k[0])) < 1e-15
    N = 9
    q, k, v = _rand((N, 6), 24), _rand((N, 6), 25), _rand((N, 6), 26)
    O, L = oracle.forward_head(q, k, v, 0.4, causal=True)
    np.testing.assert_allclose(O[0], v[0], atol=1e-15)
    assert abs(L[0] - 0.4 * float(q[0] @ k[0])) < 1e-14


def test_identical_value_rows_are_reproduced():
    N, d = 17, 5
    row = _rand((1, d), 31)
    v = np.repeat(row, N, axis=0)
    for causal in (False, True):
        O, _ = oracle.forward_head(_rand((N, d), 32), _rand((N, d), 33), v, 0.5, causal=causal)
        np.testing.assert_allclose(O, v, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_P_sum_to_one(causal):
    # with V = all ones (p = 0) every output element is the row sum of P
    N = 25
    O, _ = oracle.forward_head(_rand((N, 3), 41), _rand((N, 3), 42), np.ones((N, 2)), 1.3, causal=causal)
    np.testing.assert_allclose(O, 1.0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_shift_of_keys(causal):
    # K -> K + 1 c^T: O unchanged, LSE_i gains scale * (q_i . c)
    N, d, scale = 19, 4, 0.6
    q, k, v = _rand((N, d), 51), _rand((N, d), 52), _rand((N, d), 53)
    c = _rand((d,), 54)
    O1, L1 = oracle.forward_head(q, k, v, scale, causal=causal)
    O2, L2 = oracle.forward_head(q, k + c[None, :], v, scale, causal=causal)
    np.testing.assert_allclose(O2, O1, atol=1e-12)
    np.testing.assert_allclose(L2, L1 + scale * (q @ c), atol=1e-12)


def test_permutation_invariance_and_equivariance():
    N, d = 23, 4
    q, k, v = _rand((N, d), 61), _rand((N, d), 62), _rand((N, d), 63)
    perm = np.random.default_rng(64).permutation(N)
    O1, L1 = oracle.forward_head(q, k, v, 0.5)
    O2, L2 = oracle.forward_head(q, k[perm], v[perm], 0.5)
    np.testing.assert_allclose(O2, O1, atol=1e-13)
    np.testing.assert_allclose(L2, L1, atol=1e-13)
    O3, L3 = oracle.forward_head(q[perm], k, v, 0.5)
    np.testing.assert_allclose(O3, O1[perm], atol=1e-13)
    np.testing.assert_allclose(L3, L1[perm], atol=1e-13)


def test_block_masks_that_reduce_to_dense_and_causal():
    N, d, mb = 40, 4, 8
    q, k, v = _rand((N, d), 71), _rand((N, d), 72), _rand((N, d), 73)
    nb = N // mb
    Od, Ld = oracle.forward_head(q, k, v, 0.5)
    Ob, Lb = oracle.forward_head(q, k, v, 0.5, block_mask=np.ones((nb, nb), np.uint8), mask_block=mb)
    np.testing.assert_array_equal(Ob, Od)
    np.testing.assert_array_equal(Lb, Ld)
    Oc, Lc = oracle.forward_head(q, k, v, 0.5, causal=True)
    tril = np.tril(np.ones((nb, nb), np.uint8))
    Ot, Lt = oracle.forward_head(q, k, v, 0.5, causal=True, block_mask=tril, mask_block=mb)
    np.testing.assert_array_equal(Ot, Oc)
    np.testing.assert_array_equal(Lt, Lc)


def test_linear_in_v_and_heads_independent():
    B, H, N, d = 2, 3, 12, 4
    rng = np.random.default_rng(81)
    q, k, v1, v2 = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    O1, _ = oracle.forward(q, k, v1, 0.5, causal=True)
    O2, _ = oracle.forward(q, k, v2, 0.5, causal=True)
    O3, _ = oracle.forward(q, k, 2.0 * v1 - 3.0 * v2, 0.5, causal=True)
    np.testing.assert_allclose(O3, 2.0 * O1 - 3.0 * O2, atol=1e-12)
    # slice (1, 2) alone equals the same slice of the batched call
    Oh, Lh = oracle.forward_head(q[1, 2], k[1, 2], v1[1, 2], 0.5, causal=True, b=1, h=2)
    np.testing.assert_array_equal(O1[1, 2], Oh)


def test_forward_rows_equals_full_rows():
    B, H, N, d = 1, 2, 30, 8
    rng = np.random.default_rng(91)
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    O, L = oracle.forward(q, k, v, 0.3, causal=True, dropout_p=0.2, seed=5)
    rows = [0, 7, 29]
    Or, Lr = oracle.forward_rows(q, k, v, 0.3, 0, 1, rows, causal=True, dropout_p=0.2, seed=5)
    np.testing.assert_allclose(Or, O[0, 1, rows], atol=1e-14)
    np.testing.assert_allclose(Lr, L[0, 1, rows], atol=1e-14)


def test_accepts_bf16_torch_inputs_exactly():
    t = torch.randn(1, 1, 8, 4).to(torch.bfloat16)
    O, L = oracle.forward(t, t, t, 0.5)
    O2, L2 = oracle.forward(t.double().numpy(), t.double().numpy(), t.double().numpy(), 0.5)
    np.testing.assert_array_equal(O, O2)
