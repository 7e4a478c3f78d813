"""Exact softmax attention in float64, materializing S and P (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Forward, per (b, h) slice with Q, K, V of N rows and d columns (notation of
the FlashAttention milestone page, section "The idea": S = Q K^T,
P = softmax(S), O = P V; step order matrix product, mask, softmax, dropout,
matrix product from the same section's paragraph on the fused kernel):

    S_ij     = scale * sum_c Q_ic K_jc
    valid_ij = (not causal or j <= i) and (no block mask or bm[i // mb][j // mb] != 0)
    LSE_i    = log sum_{valid j} exp(S_ij)            (-inf when row i has no valid j)
    P_ij     = exp(S_ij - LSE_i) on valid entries, 0 elsewhere
    Pd_ij    = P_ij * Z_ij / (1 - p)                  (Z = dropout keep bits)
    O_i      = sum_j Pd_ij V_j

The block mask skips whole blocks that a fixed pattern marks empty (the
block-sparse variant in the same section). The pages keep, per query row,
the output and the two softmax statistics (running maximum and sum); the
single log-sum-exp LSE_i = m_i + log(l_i) carries the same information.

Backward, given dO (chain rule on the forward definition; the pages only
say the backward recomputes S and P from the stored statistics, FlashAttention
milestone page, "The idea", recomputation paragraph):

    dV_j  = sum_i Pd_ij dO_i
    dP_ij = (dO_i . V_j) * Z_ij / (1 - p)
    D_i   = sum_j P_ij dP_ij
    dS_ij = P_ij (dP_ij - D_i)
    dQ_i  = scale * sum_j dS_ij K_j
    dK_j  = scale * sum_i dS_ij Q_i
"""
from __future__ import annotations

import numpy as np

from .dropout_hash import dropout_keep


def _f64(x):
    """Exact upcast of a torch tensor or array to a float64 numpy array."""
    if hasattr(x, "detach"):
        x = x.detach().cpu()
        import torch

        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def valid_mask(N: int, causal: bool, block_mask=None, mask_block: int = 128, rows=None, M: int | None = None,
               cols=None):
    """Bool ``[len(rows)][len(cols)]``: which (query i, key j) pairs take part.

    ``rows`` defaults to all N query rows; ``cols`` to all ``M`` keys (``M``
    defaults to N). Causal masking is square and top-left aligned: key j is
    hidden from query i when j > i.
    """
    M = N if M is None else M
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    cols = np.arange(M) if cols is None else np.asarray(cols, dtype=np.int64)
    valid = np.ones((rows.size, cols.size), dtype=bool)
    if causal:
        valid &= cols[None, :] <= rows[:, None]
    if block_mask is not None:
        bm = np.asarray(block_mask) != 0
        valid &= bm[(rows // mask_block)[:, None], (cols // mask_block)[None, :]]
    return valid


def _probabilities(q, k, scale, valid):
    """S, LSE and P for the given query rows (q: [r][d], k: [M][d])."""
    S = scale * (q @ k.T)
    Sm = np.where(valid, S, -np.inf)
    m = Sm.max(axis=1)
    has = np.isfinite(m)
    m_safe = np.where(has, m, 0.0)
    with np.errstate(invalid="ignore", divide="ignore"):
        lse = np.where(has, m_safe + np.log(np.exp(Sm - m_safe[:, None]).sum(axis=1)), -np.inf)
    lse_safe = np.where(has, lse, 0.0)
    P = np.where(valid & has[:, None], np.exp(Sm - lse_safe[:, None]), 0.0)
    return S, lse, P


def forward_head(q, k, v, scale, causal=False, dropout_p=0.0, seed=0, b=0, h=0,
                 block_mask=None, mask_block=128, rows=None):
    """Forward of one (b, h) slice. q: [N][d] (or the rows listed in ``rows``),
    k, v: [N][d]. Returns (O [r][d], LSE [r]) in float64."""
    k = _f64(k)
    v = _f64(v)
    N = k.shape[0]
    rows_idx = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    q = _f64(q)
    if rows is not None and q.shape[0] == N:
        q = q[rows_idx]
    valid = valid_mask(N, causal, block_mask, mask_block, rows_idx)
    _, lse, P = _probabilities(q, k, scale, valid)
    if dropout_p > 0.0:
        Z = dropout_keep(seed, b, h, rows_idx, np.arange(N), dropout_p)
        P = P * Z / (1.0 - dropout_p)
    return P @ v, lse


def backward_head(q, k, v, do, scale, causal=False, dropout_p=0.0, seed=0, b=0, h=0,
                  block_mask=None, mask_block=128):
    """Backward of one (b, h) slice; every input [N][d]. Returns dict with
    dq, dk, dv ([N][d]) and D ([N]) in float64."""
    q, k, v, do = (_f64(t) for t in (q, k, v, do))
    N = q.shape[0]
    valid = valid_mask(N, causal, block_mask, mask_block)
    _, _, P = _probabilities(q, k, scale, valid)
    if dropout_p > 0.0:
        Zs = dropout_keep(seed, b, h, np.arange(N), np.arange(N), dropout_p) / (1.0 - dropout_p)
    else:
        Zs = 1.0
    Pd = P * Zs
    dv = Pd.T @ do
    dP = (do @ v.T) * Zs
    D = (P * dP).sum(axis=1)
    dS = P * (dP - D[:, None])
    dq = scale * (dS @ k)
    dk = scale * (dS.T @ q)
    return {"dq": dq, "dk": dk, "dv": dv, "D": D}


def forward(q, k, v, scale, causal=False, dropout_p=0.0, seed=0, block_mask=None,
            mask_block=128, heads=None):
    """Forward over [B][H][N][d] inputs. Returns (O [B][H][N][d], LSE [B][H][N]).

    ``heads``: optional list of (b, h) to compute; other slices are left NaN.
    """
    B, H, N, d = q.shape
    O = np.full((B, H, N, d), np.nan)
    L = np.full((B, H, N), np.nan)
    for b in range(B):
        for h in range(H):
            if heads is not None and (b, h) not in heads:
                continue
            O[b, h], L[b, h] = forward_head(q[b, h], k[b, h], v[b, h], scale, causal, dropout_p,
                                            seed, b, h, block_mask, mask_block)
    return O, L


def backward(q, k, v, do, scale, causal=False, dropout_p=0.0, seed=0, block_mask=None,
             mask_block=128, heads=None):
    """Backward over [B][H][N][d] inputs. Returns (dQ, dK, dV) in float64
    (slices outside ``heads`` are left NaN)."""
    B, H, N, d = q.shape
    out = [np.full((B, H, N, d), np.nan) for _ in range(3)]
    for b in range(B):
        for h in range(H):
            if heads is not None and (b, h) not in heads:
                continue
            g = backward_head(q[b, h], k[b, h], v[b, h], do[b, h], scale, causal, dropout_p,
                              seed, b, h, block_mask, mask_block)
            out[0][b, h], out[1][b, h], out[2][b, h] = g["dq"], g["dk"], g["dv"]
    return tuple(out)


def forward_rows(q, k, v, scale, b, h, rows, causal=False, dropout_p=0.0, seed=0,
                 block_mask=None, mask_block=128):
    """O and LSE of selected query rows of head (b, h) of [B][H][N][d] inputs,
    each row computed from its own definition (for spot checks at large N)."""
    return forward_head(q[b, h], k[b, h], v[b, h], scale, causal, dropout_p, seed, b, h,
                        block_mask, mask_block, rows=rows)


def backward_rows(q, k, v, do, scale, b, h, rows, causal=False, dropout_p=0.0, seed=0,
                  block_mask=None, mask_block=128):
    """dQ of selected query rows of head (b, h) of [B][H][N][d] inputs. Row i
    of dQ needs only row i of P and dP and D_i, so each row follows from its
    own definition: dQ_i = scale * sum_j P_ij (dP_ij - D_i) K_j."""
    rows = np.asarray(rows, dtype=np.int64)
    qh, kh, vh, doh = (_f64(t[b, h]) for t in (q, k, v, do))
    N = kh.shape[0]
    valid = valid_mask(N, causal, block_mask, mask_block, rows)
    _, _, P = _probabilities(qh[rows], kh, scale, valid)
    dP = doh[rows] @ vh.T
    if dropout_p > 0.0:
        dP = dP * dropout_keep(seed, b, h, rows, np.arange(N), dropout_p) / (1.0 - dropout_p)
    D = (P * dP).sum(axis=1)
    return scale * ((P * (dP - D[:, None])) @ kh)


def backward_cols(q, k, v, do, scale, b, h, cols, causal=False, dropout_p=0.0, seed=0,
                  block_mask=None, mask_block=128, row_chunk=256):
    """dK and dV of selected keys of head (b, h) of [B][H][N][d] inputs.

    Key j's gradients sum over the rows i that see it, and each term needs
    that row's full statistics (its LSE and D_i), so every such row is
    computed whole from the definition:

        dV_j = sum_i Pd_ij dO_i,   dK_j = scale * sum_i P_ij (dP_ij - D_i) Q_i

    The sum over i runs over the rows in increasing order, ``row_chunk`` rows
    at a time (the chunks only bound memory). Returns (dK [c][d], dV [c][d]).
    """
    cols = np.asarray(cols, dtype=np.int64)
    qh, kh, vh, doh = (_f64(t[b, h]) for t in (q, k, v, do))
    N, d = kh.shape
    seen = valid_mask(N, causal, block_mask, mask_block, cols=cols).any(axis=1)
    rows_all = np.nonzero(seen)[0]
    dk = np.zeros((cols.size, d))
    dv = np.zeros((cols.size, d))
    for c0 in range(0, rows_all.size, row_chunk):
        rows = rows_all[c0:c0 + row_chunk]
        valid = valid_mask(N, causal, block_mask, mask_block, rows)
        _, _, P = _probabilities(qh[rows], kh, scale, valid)
        dP = doh[rows] @ vh.T
        if dropout_p > 0.0:
            Zs = dropout_keep(seed, b, h, rows, np.arange(N), dropout_p) / (1.0 - dropout_p)
        else:
            Zs = 1.0
        dP = dP * Zs
        D = (P * dP).sum(axis=1)
        Pc = P[:, cols]
        dv += (Pc * (Zs[:, cols] if dropout_p > 0.0 else 1.0)).T @ doh[rows]
        dk += scale * ((Pc * (dP[:, cols] - D[:, None])).T @ qh[rows])
    return dk, dv
