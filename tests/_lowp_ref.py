"""The textbook attention algorithm run in a 16-bit input precision, on the
CPU: S, P, dP and dS are each rounded to the input dtype (as a standard
implementation stores them), products accumulate in fp32. Its error against
the fp64 oracle calibrates the tolerance of 16-bit GPU results on inputs
beyond the five workloads (peaky rows, strong dropout scaling), where a fixed
bound would not follow the size of the gradients.

Masks and dropout keep bits come from the oracle's definitions, so both
sides compute the same function."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle


def lowp_attention(q, k, v, do, scale, causal=False, dropout_p=0.0, seed=0, block_mask=None, mask_block=128):
    """(O, dQ, dK, dV) as float64 arrays; q, k, v, do are [B][H][N][d] CPU tensors."""
    B, H, N, d = q.shape
    dt = q.dtype
    out = [np.zeros((B, H, N, d)) for _ in range(4)]
    valid = torch.from_numpy(oracle.valid_mask(N, causal, block_mask, mask_block))
    for b in range(B):
        for h in range(H):
            qh, kh, vh, doh = (t[b, h].float() for t in (q, k, v, do))
            s = (scale * (qh @ kh.T)).to(dt).float()
            s = s.masked_fill(~valid, -math.inf)
            m = s.max(dim=1, keepdim=True).values
            m = torch.where(torch.isfinite(m), m, torch.zeros_like(m))
            e = torch.exp(s - m)
            den = e.sum(dim=1, keepdim=True)
            p = torch.where(den > 0, e / den.clamp_min(1e-300), torch.zeros_like(e)).to(dt).float()
            if dropout_p > 0:
                z = torch.from_numpy(oracle.dropout_keep(seed, b, h, np.arange(N), np.arange(N), dropout_p))
                zs = z.float() / (1.0 - dropout_p)
            else:
                zs = torch.ones_like(p)
            pd = (p * zs).to(dt).float()
            o = pd @ vh
            dv = pd.T @ doh
            dp = ((doh @ vh.T) * zs).to(dt).float()
            D = (p * dp).sum(dim=1, keepdim=True)
            ds = (p * (dp - D)).to(dt).float()
            dq = scale * (ds @ kh)
            dk = scale * (ds.T @ qh)
            for i, t in enumerate((o, dq, dk, dv)):
                out[i][b, h] = t.to(dt).double().numpy()
    return out
