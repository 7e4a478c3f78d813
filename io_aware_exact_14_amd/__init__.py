"""Tiled exact softmax attention for AMD MI355X (gfx950).

Python binding of libfa.so (C ABI in include/fa.h). This module only
marshals arguments: every step of forward, backward and dropout-mask
generation runs in the library's HIP kernels, on the caller's current HIP
stream. PyTorch provides device memory and streams. If the library is not
built, importing this package raises OSError.

    o, lse = forward(q, k, v, causal=True)
    dq, dk, dv = backward(q, k, v, o, lse, do, causal=True)
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional

import torch

from . import _lib
from ._lib import FA_BF16, FA_F16, FA_F32, FaParams, STATUS_NAMES

_lib.load()

__all__ = ["forward", "backward", "backward_noalloc", "backward_dq", "backward_dkdv", "dropout_mask",
           "bwd_workspace_bytes", "FaError", "params"]

_DT = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = _lib.load()
        msg = lib.fa_status_string(status).decode()
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({msg})")
        self.status = status


def _check(status: int, where: str):
    if status != 0:
        raise FaError(status, where)


def params(B, H, N, d, dtype=torch.bfloat16, *, grad_dtype=torch.float32, scale=None, causal=False,
           dropout_p=0.0, seed=0, block_mask: Optional[torch.Tensor] = None, mask_block=128) -> FaParams:
    p = FaParams()
    p.B, p.H, p.N, p.d = int(B), int(H), int(N), int(d)
    p.in_dtype = _DT[dtype]
    p.grad_dtype = _DT[grad_dtype]
    p.scale = float(1.0 / math.sqrt(d) if scale is None else scale)
    p.causal = 1 if causal else 0
    p.dropout_p = float(dropout_p)
    p.seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    p.block_mask = None if block_mask is None else block_mask.data_ptr()
    p.mask_block = int(mask_block)
    return p


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _require(t: torch.Tensor, name: str, shape, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _mask_arg(block_mask, N, mask_block, device):
    if block_mask is None:
        return None
    bm = torch.as_tensor(block_mask)
    nb = (N + mask_block - 1) // mask_block
    if tuple(bm.shape) != (nb, nb):
        raise ValueError(f"block_mask must be [{nb}][{nb}] for N={N}, mask_block={mask_block}")
    return bm.to(device=device, dtype=torch.uint8).contiguous()


def forward(q, k, v, *, scale=None, causal=False, dropout_p=0.0, seed=0, block_mask=None, mask_block=128,
            out=None, lse=None):
    """O and LSE of exact attention; q, k, v are [B][H][N][d] device tensors."""
    B, H, N, d = q.shape
    _require(q, "q", (B, H, N, d))
    _require(k, "k", (B, H, N, d), q.dtype)
    _require(v, "v", (B, H, N, d), q.dtype)
    bm = _mask_arg(block_mask, N, mask_block, q.device)
    p = params(B, H, N, d, q.dtype, scale=scale, causal=causal, dropout_p=dropout_p, seed=seed,
               block_mask=bm, mask_block=mask_block)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _require(out, "out", (B, H, N, d), q.dtype)
    _require(lse, "lse", (B, H, N), torch.float32)
    lib = _lib.load()
    _check(lib.fa_fwd(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                      _stream()), "fa_fwd")
    return out, lse


def bwd_workspace_bytes(B, H, N, d, dtype=torch.bfloat16, **kw) -> int:
    p = params(B, H, N, d, dtype, **kw)
    return int(_lib.load().fa_bwd_workspace_bytes(ctypes.byref(p)))


def _bwd_setup(q, k, v, o, lse, do, scale, causal, dropout_p, seed, block_mask, mask_block, grad_dtype, workspace):
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("do", do)) + ((("o", o),) if o is not None else ()):
        _require(t, name, (B, H, N, d), q.dtype)
    _require(lse, "lse", (B, H, N), torch.float32)
    bm = _mask_arg(block_mask, N, mask_block, q.device)
    p = params(B, H, N, d, q.dtype, grad_dtype=grad_dtype, scale=scale, causal=causal, dropout_p=dropout_p,
               seed=seed, block_mask=bm, mask_block=mask_block)
    lib = _lib.load()
    need = int(lib.fa_bwd_workspace_bytes(ctypes.byref(p)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    return p, bm, lib, workspace


def _grad(t, name, shape, grad_dtype, device):
    if t is None:
        t = torch.empty(shape, dtype=grad_dtype, device=device)
    _require(t, name, shape, grad_dtype)
    return t


def _ws(workspace):
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def backward(q, k, v, o, lse, do, *, scale=None, causal=False, dropout_p=0.0, seed=0, block_mask=None,
             mask_block=128, grad_dtype=torch.float32, workspace=None, dq=None, dk=None, dv=None):
    """dQ, dK, dV of exact attention (recomputes S and P from q, k and lse)."""
    p, bm, lib, workspace = _bwd_setup(q, k, v, o, lse, do, scale, causal, dropout_p, seed, block_mask,
                                       mask_block, grad_dtype, workspace)
    dq, dk, dv = (_grad(t, n, q.shape, grad_dtype, q.device) for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")))
    _check(lib.fa_bwd(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), *_ws(workspace), _stream()),
           "fa_bwd")
    return dq, dk, dv


def backward_noalloc(q, k, v, o, lse, do, *, dq, dk, dv, scale=None, causal=False, dropout_p=0.0, seed=0,
                     block_mask=None, mask_block=128, grad_dtype=torch.float32):
    """dQ, dK, dV through fa_bwd_noalloc: no workspace and no allocation (the
    library keeps D in a fixed per-GPU array; B*H*N up to
    _lib.BWD_NOALLOC_MAX_ROWS). The gradients are caller-provided; a block
    mask should already be a contiguous uint8 device tensor."""
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _require(t, name, (B, H, N, d), q.dtype)
    _require(lse, "lse", (B, H, N), torch.float32)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _require(t, name, (B, H, N, d), grad_dtype)
    bm = _mask_arg(block_mask, N, mask_block, q.device)
    p = params(B, H, N, d, q.dtype, grad_dtype=grad_dtype, scale=scale, causal=causal, dropout_p=dropout_p,
               seed=seed, block_mask=bm, mask_block=mask_block)
    _check(_lib.load().fa_bwd_noalloc(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                      lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                      _stream()), "fa_bwd_noalloc")
    return dq, dk, dv


def backward_dq(q, k, v, o, lse, do, *, workspace, scale=None, causal=False, dropout_p=0.0, seed=0,
                block_mask=None, mask_block=128, grad_dtype=torch.float32, dq=None):
    """First backward stage: D_i = dO_i . O_i into ``workspace``, and dQ."""
    p, bm, lib, workspace = _bwd_setup(q, k, v, o, lse, do, scale, causal, dropout_p, seed, block_mask,
                                       mask_block, grad_dtype, workspace)
    dq = _grad(dq, "dq", q.shape, grad_dtype, q.device)
    _check(lib.fa_bwd_dq(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                         do.data_ptr(), dq.data_ptr(), *_ws(workspace), _stream()), "fa_bwd_dq")
    return dq


def backward_dkdv(q, k, v, lse, do, *, workspace, scale=None, causal=False, dropout_p=0.0, seed=0,
                  block_mask=None, mask_block=128, grad_dtype=torch.float32, dk=None, dv=None):
    """Second backward stage (after backward_dq with the same workspace): dK, dV."""
    p, bm, lib, workspace = _bwd_setup(q, k, v, None, lse, do, scale, causal, dropout_p, seed, block_mask,
                                       mask_block, grad_dtype, workspace)
    dk, dv = (_grad(t, n, q.shape, grad_dtype, q.device) for t, n in ((dk, "dk"), (dv, "dv")))
    _check(lib.fa_bwd_dkdv(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(), lse.data_ptr(),
                           do.data_ptr(), dk.data_ptr(), dv.data_ptr(), *_ws(workspace), _stream()), "fa_bwd_dkdv")
    return dk, dv


def dropout_mask(B, H, N, d, b, h, i0, rows, j0, cols, *, dropout_p, seed, dtype=torch.bfloat16,
                 device="cuda"):
    """Keep bits (uint8 [rows][cols], 1 = kept) of head (b, h) from the device hash."""
    p = params(B, H, N, d, dtype, dropout_p=dropout_p, seed=seed)
    keep = torch.empty((rows, cols), dtype=torch.uint8, device=device)
    _check(_lib.load().fa_dropout_mask(ctypes.byref(p), b, h, i0, rows, j0, cols, keep.data_ptr(), _stream()),
           "fa_dropout_mask")
    return keep
