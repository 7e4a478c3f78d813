"""Parity at the workloads' full sizes, in the launch configuration bench.py
times (fp32 gradients), against the fp64 oracle: every output element of
one or two whole heads, plus sampled query rows (O, LSE, dQ) and sampled
keys (dK, dV) of three further heads, plus properties that hold at any size.

Each workload prints one line `PARITY {json}` with, per tensor, the max-abs
error and the 99.9th percentile of the absolute error over every element
compared, and the number of elements."""
import json
import math

import numpy as np
import pytest
import torch

import oracle
from tests._gpu import TOL, note
from workloads import WORKLOADS, workload_inputs

pytestmark = pytest.mark.gpu

# (workload, heads compared in full, heads compared on sampled rows and keys)
CASES = [
    ("C1", [(0, 0)], []),
    ("C2", [(0, 0), (7, 15)], [(2, 3), (5, 9), (6, 0)]),
    ("C3", [(3, 15)], [(0, 0), (1, 7), (2, 11)]),
    ("C4", [(0, 31)], [(0, 0), (0, 13), (0, 22)]),
    ("C5", [(1, 15)], [(0, 0), (1, 4), (0, 9)]),
]


def _run(fa, w, x):
    dev = torch.device("cuda:0")
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    bm = torch.from_numpy(x["block_mask"]) if x["block_mask"] is not None else None
    kw = dict(scale=w.scale, causal=w.causal, dropout_p=w.dropout_p, seed=w.dropout_seed, block_mask=bm,
              mask_block=w.mask_block)
    o, lse = fa.forward(q, k, v, **kw)
    grads = None
    if w.backward:
        grads = fa.backward(q, k, v, o, lse, x["do"].to(dev), grad_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    out = {"o": o.float().cpu().numpy(), "lse": lse.cpu().numpy()}
    if grads is not None:
        out.update({n: g.cpu().numpy() for n, g in zip(("dq", "dk", "dv"), grads)})
    return out


def _abs_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    both_inf = np.isinf(got) & np.isinf(ref) & (np.sign(got) == np.sign(ref))
    with np.errstate(invalid="ignore"):
        d = np.where(both_inf, 0.0, np.abs(got - ref))
    return np.where(np.isnan(d), np.inf, d).ravel()


def _sample_keys(w, rng):
    """16 keys of a head: uniform over the sequence, except at 16K tokens,
    where a causal key near the start is seen by every later row (a whole
    head's work in the oracle): there they come from the last 2048 keys."""
    lo = w.N - 2048 if w.N > 8192 else 0
    keys = np.sort(rng.choice(np.arange(lo, w.N), size=16, replace=False))
    keys[-1] = w.N - 1
    return keys


@pytest.mark.parametrize("name,full_heads,sampled_heads", CASES, ids=[c[0] for c in CASES])
def test_workload_full_size(fa, name, full_heads, sampled_heads):
    w = WORKLOADS[name]
    x = workload_inputs(w)
    note(f"workload {name} full size: B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype}")
    out = _run(fa, w, x)
    tol = TOL[w.torch_dtype]
    bm = x["block_mask"]
    errs = {n: [] for n in ("O", "LSE", "dQ", "dK", "dV")}
    cargs = (w.causal, w.dropout_p, w.dropout_seed)
    for (b, h) in full_heads:
        O, L = oracle.forward_head(x["q"][b, h], x["k"][b, h], x["v"][b, h], w.scale, *cargs, b, h, bm,
                                   w.mask_block)
        errs["O"].append(_abs_err(out["o"][b, h], O))
        errs["LSE"].append(_abs_err(out["lse"][b, h], L))
        if w.backward:
            g = oracle.backward_head(x["q"][b, h], x["k"][b, h], x["v"][b, h], x["do"][b, h], w.scale, *cargs,
                                     b, h, bm, w.mask_block)
            for n, key in (("dQ", "dq"), ("dK", "dk"), ("dV", "dv")):
                errs[n].append(_abs_err(out[key][b, h], g[key]))
    rng = np.random.default_rng(99)
    for (b, h) in sampled_heads:
        rows = np.sort(rng.choice(w.N, size=min(16, w.N), replace=False))
        rows[-1] = w.N - 1  # the last row (tail / longest causal row)
        O, L = oracle.forward_rows(x["q"], x["k"], x["v"], w.scale, b, h, rows, *cargs, bm, w.mask_block)
        errs["O"].append(_abs_err(out["o"][b, h][rows], O))
        errs["LSE"].append(_abs_err(out["lse"][b, h][rows], L))
        if w.backward:
            dq = oracle.backward_rows(x["q"], x["k"], x["v"], x["do"], w.scale, b, h, rows, *cargs, bm,
                                      w.mask_block)
            errs["dQ"].append(_abs_err(out["dq"][b, h][rows], dq))
            keys = _sample_keys(w, rng)
            dk, dv = oracle.backward_cols(x["q"], x["k"], x["v"], x["do"], w.scale, b, h, keys, *cargs, bm,
                                          w.mask_block)
            errs["dK"].append(_abs_err(out["dk"][b, h][keys], dk))
            errs["dV"].append(_abs_err(out["dv"][b, h][keys], dv))
    report = {"workload": name, "tolerance": tol, "full_heads": [list(t) for t in full_heads],
              "sampled_heads": [list(t) for t in sampled_heads]}
    for n, parts in errs.items():
        if not parts:
            continue
        e = np.concatenate(parts)
        report[n] = {"max_abs": float(e.max()), "p999": float(np.quantile(e, 0.999)), "n": int(e.size)}
    print("PARITY " + json.dumps(report), flush=True)
    for n in errs:
        if n in report:
            assert report[n]["max_abs"] <= tol, (name, n, report[n])
    # properties at any size: every row has a valid key, so everything is finite
    assert np.isfinite(out["o"]).all() and np.isfinite(out["lse"]).all()
    if w.backward:
        for n in ("dq", "dk", "dv"):
            assert np.isfinite(out[n]).all(), n
        # softmax is shift invariant per row, so sum over keys of dK is 0 in
        # exact arithmetic; with fp32 accumulation it is small next to |dK|
        s = np.abs(out["dk"].sum(axis=2)).max()
        assert s <= 1e-2 * math.sqrt(w.N) * max(1.0, float(np.abs(out["dk"]).max())), s
