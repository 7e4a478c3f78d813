"""The Python binding without a GPU: argument marshalling (the parameter
block it builds, workspace size, status-to-exception mapping) and its
host-side argument checks. No kernel is launched."""
import math

import pytest
import torch

from tests.test_abi import _ensure_built


@pytest.fixture(scope="module")
def fa():
    _ensure_built()
    import io_aware_exact_14_amd as fa_mod

    return fa_mod


def test_params_block(fa):
    from io_aware_exact_14_amd import _lib

    p = fa.params(2, 3, 100, 128, torch.float16, causal=True, dropout_p=0.25, seed=-1)
    assert (p.B, p.H, p.N, p.d) == (2, 3, 100, 128)
    assert p.in_dtype == _lib.FA_F16 and p.grad_dtype == _lib.FA_F32
    assert p.scale == pytest.approx(1 / math.sqrt(128))
    assert p.causal == 1 and p.dropout_p == 0.25
    assert p.seed == 2**64 - 1  # seeds are taken modulo 2^64
    assert not p.block_mask and p.mask_block == 128
    assert fa.params(1, 1, 8, 64, torch.bfloat16, scale=0.3, grad_dtype=torch.bfloat16).grad_dtype == _lib.FA_BF16


def test_workspace_bytes(fa):
    for B, H, N in ((1, 1, 1), (2, 3, 100), (8, 16, 1024)):
        assert fa.bwd_workspace_bytes(B, H, N, 64) == (B * H * N * 4 + 255) // 256 * 256
    assert fa.bwd_workspace_bytes(1, 1, 10, 96) == 0  # invalid head dimension


def test_status_becomes_exception(fa):
    err = fa.FaError(4, "fa_fwd")
    assert err.status == 4 and "FA_ERR_HEADDIM" in str(err) and "fa_fwd" in str(err)
    with pytest.raises(fa.FaError):
        fa._check(2, "where")
    fa._check(0, "where")


def test_host_tensors_are_rejected(fa):
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        fa.forward(q, q, q)
    with pytest.raises(ValueError, match="device tensor"):
        fa.backward(q, q, q, q, torch.zeros(1, 1, 8), q)


def test_block_mask_shape_is_checked(fa):
    assert fa._mask_arg(None, 300, 128, "cpu") is None
    ok = fa._mask_arg(torch.ones(3, 3, dtype=torch.bool), 300, 128, "cpu")
    assert ok.dtype == torch.uint8 and ok.is_contiguous()
    with pytest.raises(ValueError, match=r"\[3\]\[3\]"):
        fa._mask_arg(torch.ones(2, 2), 300, 128, "cpu")
