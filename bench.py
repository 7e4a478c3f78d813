#!/usr/bin/env python3
"""Throughput of tiled exact attention (forward + backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
    python bench.py --workload C2 --only           one workload (profiling runs)
    python bench.py --standard [--workload C2]     standard vs tiled attention
    python bench.py --sweep [--sweep-n 1024,...]   sequence-length sweep
    python bench.py --roofs                        MFMA / VALU / LDS / tile skeleton / HBM / launch microbenchmarks

A step is one pass of the whole hot path over one batch of synthetic input:
fa_fwd (O, LSE), then the two backward stages fa_bwd_dq (D, dQ) and
fa_bwd_dkdv (dK, dV), all through the C ABI on the current HIP stream.
Inputs are resident in device memory before the timed region. The headline
workload is the long-context layer (B=1, H=32, N=16384, d=128, bf16,
causal), the largest of the five; the same JSON line carries a `configs`
entry for each of the five workloads (C1..C5), each with forward, backward
and step TFLOP/s, MFMA fractions, warm and cache-flushed timings, per-kernel
durations and the roofline of its dominant kernel. Prints ONE JSON line on
stdout; progress goes to stderr.

FLOP convention: forward 4*B*H*N^2*d (halved when causal, kept-block count
when block-sparse), backward 2.5x forward.

Per-kernel durations come from K back-to-back launches of one kernel between
a single pair of HIP events on the launch stream, so they leave out the
gaps between dependent kernels and sum to at most the step time.
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd+bwd TFLOP/s and % MFMA peak on 1 MI355X (bf16, N=1k–16k)"
# Published MI355X peaks: dense MFMA (TFLOP/s) by operand type, HBM3E (GB/s).
PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "fp32": 157.3}
PEAK_HBM_GBS = 8000.0
DTYPE_NAME = {"bf16": "bf16", "fp16": "fp16", "fp32": "fp32"}

WORKLOAD_TEXT = {
    "C1": "single-head attention forward, fp32: B=1 H=1 N=128 d=64, non-causal",
    "C2": "GPT-2-medium attention layer fwd+bwd: B=8 H=16 N=1024 d=64 bf16 causal",
    "C3": "training-style attention fwd+bwd: B=4 H=16 N=4096 d=64 bf16 causal dropout 0.1",
    "C4": "long-context attention fwd+bwd: B=1 H=32 N=16384 d=128 bf16 causal, K x2",
    "C5": "block-sparse attention fwd+bwd: B=2 H=16 N=8192 d=64 bf16, 128x128 blocks (518/4096 kept)",
}


def src_digest() -> str:
    """sha256 over the kernel sources and the ABI header (ties profiles to code)."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "io_aware_exact_14_amd", "csrc", "*")))
    files.append(os.path.join(ROOT, "include", "fa.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def convention_flops(w, kept_blocks):
    B, H, N, d = w.B, w.H, w.N, w.d
    if w.block_sparse:
        fwd = 4.0 * B * H * d * w.mask_block ** 2 * kept_blocks
    else:
        fwd = 4.0 * B * H * N * N * d * (0.5 if w.causal else 1.0)
    return fwd, (2.5 * fwd if w.backward else 0.0)


def kernel_model(w, kept_blocks, el_bytes, grad_bytes):
    """Algorithmic flops and compulsory bytes per launch of each kernel.

    Flops: 2*d per visible (query, key) pair per matrix product the kernel's
    outputs require (forward 2: QK^T, PV; dQ 3: QK^T, dO V^T, dS K; dK/dV 4:
    QK^T, dO V^T, P^T dO, dS^T Q). Bytes: each tensor the kernel must read or
    write once (Q, K, V, O, dO, gradients, LSE and D rows)."""
    B, H, N, d = w.B, w.H, w.N, w.d
    if w.block_sparse:
        pairs = B * H * w.mask_block ** 2 * kept_blocks
    else:
        pairs = B * H * N * N * (0.5 if w.causal else 1.0)
    t = B * H * N * d  # elements of one [B][H][N][d] tensor
    rows = B * H * N
    m = {"fwd_kernel": (2 * 2 * d * pairs, 3 * t * el_bytes + t * el_bytes + 4 * rows)}
    if w.backward:
        m["bwd_dq_kernel"] = (3 * 2 * d * pairs, 5 * t * el_bytes + 4 * rows + t * grad_bytes + 4 * rows)
        m["bwd_dkdv_kernel"] = (4 * 2 * d * pairs, 4 * t * el_bytes + 8 * rows + 2 * t * grad_bytes)
    return m


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None
    when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}__{workload}__traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("src_sha256") != src_digest():
        return None
    try:
        return float(kv["traffic_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, x, target_s=20.0):
    """The fp64 oracle, as it stands, timed on the host over a bounded sample
    of the workload: whole (b, h) heads, each forward (oracle.forward_head)
    then backward (oracle.backward_head), until about ``target_s`` seconds
    have passed (at least one head). Rates follow the FLOP convention."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info

        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        cores = len(os.sched_getaffinity(0))
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    bm = x["block_mask"]
    done, t_fwd, t_bwd = 0, 0.0, 0.0
    for (b, h) in heads:
        t0 = time.perf_counter()
        oracle.forward_head(x["q"][b, h], x["k"][b, h], x["v"][b, h], w.scale, w.causal, w.dropout_p,
                            w.dropout_seed, b, h, bm, w.mask_block)
        t1 = time.perf_counter()
        if w.backward:
            oracle.backward_head(x["q"][b, h], x["k"][b, h], x["v"][b, h], x["do"][b, h], w.scale, w.causal,
                                 w.dropout_p, w.dropout_seed, b, h, bm, w.mask_block)
        t2 = time.perf_counter()
        t_fwd += t1 - t0
        t_bwd += t2 - t1
        done += 1
        if t_fwd + t_bwd >= target_s:
            break
    kept = int(np.asarray(bm).sum()) if bm is not None else 0
    f, bwd = convention_flops(w, kept)
    fh, bh = f / (w.B * w.H), bwd / (w.B * w.H)
    out = {
        "value": round((fh + bh) * done / (t_fwd + t_bwd) / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"{done} of {w.B * w.H} (b,h) heads of {w.name}, fp64 numpy, each forward then backward; "
                  f"{t_fwd:.1f} s forward + {t_bwd:.1f} s backward wall",
        "cpu_model": _cpu_model(),
        "host_threads_available": len(os.sched_getaffinity(0)),
        "fwd_value": round(fh * done / t_fwd / 1e12, 6),
    }
    if w.backward:
        out["bwd_value"] = round(bh * done / t_bwd / 1e12, 6)
        out["fwd_bwd_value"] = out["value"]
    return out


def standard_attention(q, k, v, do, scale, causal_mask=None):
    """Standard attention, forward and backward, as a chain of PyTorch/ROCm
    library kernels that write every N x N intermediate to device memory.

    This is the algorithm the tiled method is measured against (FlashAttention
    milestone page, "The idea": the standard implementation stores S and P in
    HBM). Forward: S = scale Q K^T (batched GEMM, input-dtype output), masked
    fill of S, P = softmax(S) (fp32 arithmetic inside, input-dtype storage),
    O = P V. Backward: dV^T = dO^T P, dP = dO V^T, dS = P (dP - rowsum(P dP))
    (PyTorch's fused softmax backward), dQ = scale dS K, dK^T = scale Q^T dS.
    Every product takes contiguous operands: the N x d transposes are
    materialized, the N x N matrices are never transposed. ``causal_mask`` is
    a bool [N][N] device tensor, True where a key is hidden. Returns
    (O, dQ, dK, dV) in the input dtype.
    """
    import torch

    B, H, N, d = q.shape
    BH = B * H
    q3, k3, v3, do3 = (t.reshape(BH, N, d) for t in (q, k, v, do))
    dt, dev = q.dtype, q.device
    s = torch.empty(BH, N, N, dtype=dt, device=dev).baddbmm_(q3, k3.transpose(1, 2).contiguous(),
                                                             beta=0.0, alpha=scale)
    if causal_mask is not None:
        s.masked_fill_(causal_mask, float("-inf"))
    p = torch.softmax(s, dim=-1)
    del s
    o = torch.bmm(p, v3)
    dvT = torch.bmm(do3.transpose(1, 2).contiguous(), p)
    dp = torch.bmm(do3, v3.transpose(1, 2).contiguous())
    ds = torch._softmax_backward_data(dp, p, -1, dt)
    del dp, p
    dq = torch.empty(BH, N, d, dtype=dt, device=dev).baddbmm_(ds, k3, beta=0.0, alpha=scale)
    dkT = torch.empty(BH, d, N, dtype=dt, device=dev).baddbmm_(q3.transpose(1, 2).contiguous(), ds,
                                                               beta=0.0, alpha=scale)
    shape = (B, H, N, d)
    return (o.reshape(shape), dq.reshape(shape), dkT.transpose(1, 2).reshape(shape),
            dvT.transpose(1, 2).reshape(shape))


def _tiled_step_fn(lib, p, q, k, v, do, o, lse, dq, dk, dv, ws, stream):
    """One fwd + bwd pass through the C ABI (fa_fwd, fa_bwd_dq, fa_bwd_dkdv)."""
    sp = ctypes.c_void_p(stream.cuda_stream)
    pp = ctypes.byref(p)
    fwd_args = (pp, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), sp)
    dq_args = (pp, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
               dq.data_ptr(), ws.data_ptr(), ws.numel(), sp)
    dkdv_args = (pp, q.data_ptr(), k.data_ptr(), v.data_ptr(), lse.data_ptr(), do.data_ptr(), dk.data_ptr(),
                 dv.data_ptr(), ws.data_ptr(), ws.numel(), sp)

    def fwd():
        if lib.fa_fwd(*fwd_args) != 0:
            raise RuntimeError("fa_fwd failed")

    def bwd():
        if lib.fa_bwd_dq(*dq_args) != 0 or lib.fa_bwd_dkdv(*dkdv_args) != 0:
            raise RuntimeError("fa_bwd failed")

    return fwd, bwd


def _time_fwd_bwd(fwd, bwd, steps, warmup, stream, warm_ms=0.0):
    """(ms per fwd+bwd step by wall clock, forward ms, backward ms by HIP events).
    With ``warm_ms`` > 0, untimed steps run for about that much device time
    after the warm-up steps (the clock ramps up under sustained load)."""
    import torch

    for _ in range(warmup):
        fwd()
        bwd()
    if warm_ms > 0.0:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fwd()
        bwd()
        e1.record(stream)
        torch.cuda.synchronize()
        one = max(e0.elapsed_time(e1), 1e-3)
        for _ in range(int(math.ceil(warm_ms / one))):
            fwd()
            bwd()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fwd()
        bwd()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in ev:
        e[0].record(stream)
        fwd()
        e[1].record(stream)
        bwd()
        e[2].record(stream)
    torch.cuda.synchronize()
    f = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    b = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    return ms, f, b


def _peak_extra_bytes(run):
    """Device memory a call allocates at its peak beyond what is already resident."""
    import torch

    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    out = run()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    del out
    return int(peak)


def read_step_traffic(workload: str):
    """HBM bytes per fwd+bwd step of the standard and the tiled path from the
    committed rocprofv3 counter summary ({} when absent; the tiled figure only
    while the kernel sources are unchanged)."""
    path = os.path.join(ROOT, "profiles", f"standard_vs_tiled__{workload}__traffic.txt")
    if not os.path.exists(path):
        return {}
    kv = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    out = {}
    try:
        out["standard"] = float(kv["standard_bytes_per_step"])
        if kv.get("src_sha256") == src_digest():
            out["tiled"] = float(kv["tiled_bytes_per_step"])
    except (KeyError, ValueError):
        pass
    return out


def run_standard(args):
    """Standard vs tiled attention on one workload (no dropout, no block mask):
    fwd/bwd time, convention TFLOP/s, peak extra device memory, and HBM bytes
    per step from the committed counter summary."""
    import numpy as np
    import torch

    import io_aware_exact_14_amd as fa
    from io_aware_exact_14_amd import _lib
    from workloads import WORKLOADS, workload_inputs

    w = WORKLOADS[args.workload]
    if w.dropout_p > 0 or w.block_sparse or not w.backward:
        print(f"--standard covers dense workloads with a backward pass (no dropout, no block mask); "
              f"{w.name} is not one", file=sys.stderr)
        return 2
    x = workload_inputs(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
    stream = torch.cuda.current_stream()
    lib = _lib.load()
    p = fa.params(w.B, w.H, w.N, w.d, w.torch_dtype, scale=w.scale, causal=w.causal)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in range(3))
    ws = torch.empty(max(int(lib.fa_bwd_workspace_bytes(ctypes.byref(p))), 1), dtype=torch.uint8, device=dev)
    t_fwd, t_bwd = _tiled_step_fn(lib, p, q, k, v, do, o, lse, dq, dk, dv, ws, stream)
    mask = (torch.ones(w.N, w.N, dtype=torch.bool).triu_(1).to(dev)) if w.causal else None

    if args.copy_calibration:
        src = torch.ones(512 * 2**20 // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    holder = {}

    def s_fwd_bwd():
        holder["out"] = standard_attention(q, k, v, do, w.scale, mask)

    def nothing():
        pass

    f_fwd, f_bwd = convention_flops(w, 0)
    res = {}
    ms, fm, bm = _time_fwd_bwd(t_fwd, t_bwd, args.steps, args.warmup, stream)
    res["tiled"] = {"ms_per_step": round(ms, 5), "fwd_ms": round(fm, 5), "bwd_ms": round(bm, 5)}
    # the standard chain is one function; time it whole (events bracket it)
    ms_s, _, _ = _time_fwd_bwd(s_fwd_bwd, nothing, args.steps, args.warmup, stream)
    res["standard"] = {"ms_per_step": round(ms_s, 5)}
    holder.clear()
    for name, r in res.items():
        r["tflops"] = round((f_fwd + f_bwd) / (r["ms_per_step"] * 1e-3) / 1e12, 3)
    del o, lse, dq, dk, dv, ws
    res["tiled"]["peak_extra_bytes"] = _peak_extra_bytes(
        lambda: (fa.backward(q, k, v, *fa.forward(q, k, v, scale=w.scale, causal=w.causal), do,
                             scale=w.scale, causal=w.causal)))
    res["standard"]["peak_extra_bytes"] = _peak_extra_bytes(lambda: standard_attention(q, k, v, do, w.scale, mask))
    traffic = read_step_traffic(w.name)
    for name in res:
        res[name]["hbm_bytes_per_step"] = traffic.get(name)
    line = {
        "metric": "standard vs tiled attention, fwd+bwd on 1 MI355X",
        "workload": f"{w.name}: {WORKLOAD_TEXT[w.name]}",
        "dtype": DTYPE_NAME[w.dtype],
        "data": "synthetic",
        "steps": args.steps,
        "warmup": args.warmup,
        "convention_gflop_per_step": round((f_fwd + f_bwd) / 1e9, 3),
        "standard_computes": "full N x N products (the causal mask is applied after the GEMM); "
                             "outputs and gradients in the input dtype",
        "tiled": res["tiled"],
        "standard": res["standard"],
        "speedup": round(res["standard"]["ms_per_step"] / res["tiled"]["ms_per_step"], 3),
    }
    if traffic.get("standard") and traffic.get("tiled"):
        line["hbm_ratio"] = round(traffic["standard"] / traffic["tiled"], 3)
    print(json.dumps(line), flush=True)
    return 0


def run_sweep(args):
    """Tiled attention (bf16, causal) over sequence lengths: fwd and fwd+bwd
    time, convention TFLOP/s and peak extra device memory, with standard
    attention beside it while its N x N intermediates fit the memory cap."""
    import torch

    import io_aware_exact_14_amd as fa
    from io_aware_exact_14_amd import _lib
    from workloads import draw_qkvdo

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    lib = _lib.load()
    rows = []
    for d in [int(t) for t in args.sweep_d.split(",")]:
        H = 1024 // d
        for N in [int(t) for t in args.sweep_n.split(",")]:
            B = max(1, args.sweep_tokens // N)
            q, k, v, do = (t.to(dev) for t in draw_qkvdo(B, H, N, d, torch.bfloat16, 4000 + N + d))
            scale = 1.0 / math.sqrt(d)
            p = fa.params(B, H, N, d, torch.bfloat16, scale=scale, causal=True)
            o = torch.empty_like(q)
            lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
            dq, dk, dv = (torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in range(3))
            ws = torch.empty(max(int(lib.fa_bwd_workspace_bytes(ctypes.byref(p))), 1), dtype=torch.uint8,
                             device=dev)
            t_fwd, t_bwd = _tiled_step_fn(lib, p, q, k, v, do, o, lse, dq, dk, dv, ws, stream)
            steps = max(3, min(args.steps, int(2e5 // N)))
            ms, fm, bm = _time_fwd_bwd(t_fwd, t_bwd, steps, max(1, min(args.warmup, 3)), stream, args.warm_ms)
            fwd_fl = 4.0 * B * H * N * N * d * 0.5
            del o, lse, dq, dk, dv, ws
            row = {"N": N, "B": B, "H": H, "d": d, "steps": steps,
                   "tiled": {"ms_per_step": round(ms, 4), "fwd_ms": round(fm, 4), "bwd_ms": round(bm, 4),
                             "fwd_tflops": round(fwd_fl / (fm * 1e-3) / 1e12, 2),
                             "bwd_tflops": round(2.5 * fwd_fl / (bm * 1e-3) / 1e12, 2),
                             "tflops": round(3.5 * fwd_fl / (ms * 1e-3) / 1e12, 2),
                             "peak_extra_bytes": _peak_extra_bytes(
                                 lambda: fa.backward(q, k, v, *fa.forward(q, k, v, causal=True), do,
                                                     causal=True))}}
            # standard attention peaks at four live N x N matrices (measured)
            need = 4 * B * H * N * N * 2
            if need <= args.standard_cap_gb * 2**30:
                mask = torch.ones(N, N, dtype=torch.bool).triu_(1).to(dev)
                holder = {}

                def s_run():
                    holder["o"] = standard_attention(q, k, v, do, scale, mask)

                sms, _, _ = _time_fwd_bwd(s_run, lambda: None, max(2, steps // 2), 1, stream)
                holder.clear()
                row["standard"] = {"ms_per_step": round(sms, 4),
                                   "tflops": round(3.5 * fwd_fl / (sms * 1e-3) / 1e12, 2),
                                   "peak_extra_bytes": _peak_extra_bytes(
                                       lambda: standard_attention(q, k, v, do, scale, mask))}
                del mask
            else:
                row["standard"] = {"skipped": f"four N x N matrices need {need / 2**30:.0f} GiB, above the "
                                              f"{args.standard_cap_gb} GiB cap"}
            print(json.dumps(row), file=sys.stderr, flush=True)
            rows.append(row)
            del q, k, v, do
            torch.cuda.empty_cache()
    print(json.dumps({"metric": "tiled attention fwd+bwd over sequence length on 1 MI355X (bf16, causal, "
                                "hidden 1024)", "data": "synthetic", "unit": "TFLOP/s", "rows": rows}), flush=True)
    return 0




# ---------------------------------------------------------------------------
# the default run: the headline workload plus one entry per workload
# ---------------------------------------------------------------------------
class _Case:
    """Device inputs, outputs and C-ABI launch closures of one workload."""

    def __init__(self, w, dev, lib):
        import numpy as np
        import torch

        import io_aware_exact_14_amd as fa
        from workloads import workload_inputs

        self.w = w
        self.x = workload_inputs(w)
        x = self.x
        self.q, self.k, self.v = (x[n].to(dev) for n in ("q", "k", "v"))
        self.do = x["do"].to(dev) if w.backward else None
        bm = x["block_mask"]
        self.kept = int(np.asarray(bm).sum()) if bm is not None else 0
        self.bm_dev = torch.from_numpy(bm).to(dev) if bm is not None else None
        self.grad_dtype = torch.float32
        self.p = fa.params(w.B, w.H, w.N, w.d, w.torch_dtype, grad_dtype=self.grad_dtype, scale=w.scale,
                           causal=w.causal, dropout_p=w.dropout_p, seed=w.dropout_seed, block_mask=self.bm_dev,
                           mask_block=w.mask_block)
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        if w.backward:
            self.dq, self.dk, self.dv = (torch.empty(self.q.shape, dtype=self.grad_dtype, device=dev)
                                         for _ in range(3))
            self.ws = torch.empty(max(int(lib.fa_bwd_workspace_bytes(ctypes.byref(self.p))), 1), dtype=torch.uint8,
                                  device=dev)
        self.stream = torch.cuda.current_stream()
        sp = ctypes.c_void_p(self.stream.cuda_stream)
        pp = ctypes.byref(self.p)
        fwd_args = (pp, self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), self.o.data_ptr(),
                    self.lse.data_ptr(), sp)
        self.launch = {"fwd_kernel": lambda: lib.fa_fwd(*fwd_args)}
        if w.backward:
            dq_args = (pp, self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), self.o.data_ptr(),
                       self.lse.data_ptr(), self.do.data_ptr(), self.dq.data_ptr(), self.ws.data_ptr(),
                       self.ws.numel(), sp)
            dkdv_args = (pp, self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), self.lse.data_ptr(),
                         self.do.data_ptr(), self.dk.data_ptr(), self.dv.data_ptr(), self.ws.data_ptr(),
                         self.ws.numel(), sp)
            self.launch["bwd_dq_kernel"] = lambda: lib.fa_bwd_dq(*dq_args)
            self.launch["bwd_dkdv_kernel"] = lambda: lib.fa_bwd_dkdv(*dkdv_args)
        self.names = list(self.launch)

    def step(self):
        st = 0
        for n in self.names:
            st |= self.launch[n]()
        if st != 0:
            raise RuntimeError(f"libfa returned status {st} on {self.w.name}")


def _roofline(w, model, kernel, avg_ms, peak_f):
    flops_k, bytes_k = model[kernel]
    sec = avg_ms * 1e-3
    if flops_k / (peak_f * 1e12) >= bytes_k / (PEAK_HBM_GBS * 1e9):
        roof = {"bound": "mfma", "achieved": round(flops_k / sec / 1e12, 3), "peak": peak_f, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(bytes_k / sec / 1e9, 3), "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 5)
    roof["kernel"] = kernel
    roof["kernel_avg_ms"] = round(avg_ms, 5)
    roof["algorithmic_flops"] = flops_k
    roof["compulsory_bytes"] = bytes_k
    roof["traffic"] = read_traffic(kernel, w.name)
    return roof


def measure(case, steps, warmup, flush_buf, warm_ms=0.0):
    """Warm whole steps by the host clock, per-kernel back-to-back durations
    and cache-flushed steps (a 512 MiB write before each) by HIP events.

    ``warmup`` steps run first; with ``warm_ms`` > 0, further untimed steps
    run until that much device time has passed, since the GPU clock climbs
    over the first tens of milliseconds of sustained load (the MFMA
    microbenchmark of ``--roofs`` runs at ~1.8 GHz over 3 ms and ~2.3 GHz
    over 23 ms)."""
    import torch

    w = case.w
    for _ in range(warmup):
        case.step()
    if warm_ms > 0.0:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(case.stream)
        case.step()
        e1.record(case.stream)
        torch.cuda.synchronize()
        one = max(e0.elapsed_time(e1), 1e-3)
        for _ in range(int(math.ceil(warm_ms / one))):
            case.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        case.step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    # the same K back-to-back steps timed on the device (one event pair)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(case.stream)
    for _ in range(steps):
        case.step()
    e1.record(case.stream)
    torch.cuda.synchronize()
    ms_step_dev = e0.elapsed_time(e1) / steps

    per_kernel = {}
    for n in case.names:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn = case.launch[n]
        fn()
        torch.cuda.synchronize()
        e0.record(case.stream)
        for _ in range(steps):
            fn()
        e1.record(case.stream)
        torch.cuda.synchronize()
        per_kernel[n] = e0.elapsed_time(e1) / steps
    # leave the outputs of one whole, ordered step behind
    case.step()

    if flush_buf is None:
        flushed = None
    else:
        flushed = []
    for i in range(steps if flush_buf is not None else 0):
        flush_buf.fill_(float(i & 7))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(case.stream)
        case.step()
        e1.record(case.stream)
        torch.cuda.synchronize()
        flushed.append(e0.elapsed_time(e1))
    ms_flushed = sorted(flushed)[len(flushed) // 2] if flushed else None

    el = torch.tensor([], dtype=w.torch_dtype).element_size()
    model = kernel_model(w, case.kept, el, torch.tensor([], dtype=case.grad_dtype).element_size())
    f_fwd, f_bwd = convention_flops(w, case.kept)
    peak_f = PEAK_TFLOPS[w.dtype]
    t_fwd = per_kernel["fwd_kernel"]
    t_bwd = sum(per_kernel[n] for n in case.names[1:])
    step_tf = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12
    entry = {
        "workload": f"{w.name}: {WORKLOAD_TEXT[w.name]}",
        "dtype": DTYPE_NAME[w.dtype],
        "steps": steps,
        "ms_per_step": round(ms_step, 5),
        "ms_per_step_device_events": round(ms_step_dev, 5),
        "tflops": round(step_tf, 3),
        "mfma_frac": round(step_tf / peak_f, 5),
        "fwd_tflops": round(f_fwd / (t_fwd * 1e-3) / 1e12, 3),
        "fwd_mfma_frac": round(f_fwd / (t_fwd * 1e-3) / 1e12 / peak_f, 5),
        "per_kernel": {n: {"avg_ms": round(per_kernel[n], 5),
                           "tflops": round(model[n][0] / (per_kernel[n] * 1e-3) / 1e12, 3),
                           "mfma_frac": round(model[n][0] / (per_kernel[n] * 1e-3) / 1e12 / peak_f, 5),
                           "gbs": round(model[n][1] / (per_kernel[n] * 1e-3) / 1e9, 1)} for n in case.names},
        "flushed": None if ms_flushed is None else {
            "ms_per_step": round(ms_flushed, 5),
            "tflops": round((f_fwd + f_bwd) / (ms_flushed * 1e-3) / 1e12, 3),
            "method": "median of K steps, each after a 512 MiB device write, HIP events around the step"},
    }
    if w.backward:
        entry["bwd_tflops"] = round(f_bwd / (t_bwd * 1e-3) / 1e12, 3)
        entry["bwd_mfma_frac"] = round(f_bwd / (t_bwd * 1e-3) / 1e12 / peak_f, 5)
    dom = max(case.names, key=lambda n: per_kernel[n])
    entry["roofline"] = _roofline(w, model, dom, per_kernel[dom], peak_f)
    return entry


def run_main(args):
    import torch

    from io_aware_exact_14_amd import _lib
    from workloads import WORKLOADS

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = _lib.load()
    order = [args.workload] if args.only else [args.workload] + [n for n in sorted(WORKLOADS) if n != args.workload]
    flush_buf = None if args.no_flush else torch.empty(512 * 2**20 // 4, dtype=torch.float32, device=dev)
    if args.copy_calibration:
        src = torch.ones(512 * 2**20 // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    entries = {}
    head_case_x = None
    for name in order:
        w = WORKLOADS[name]
        t0 = time.perf_counter()
        case = _Case(w, dev, lib)
        # the headline takes exactly --steps/--warmup; the small workloads take
        # at least 100 steps so their microsecond kernels average over enough launches
        is_head = name == args.workload
        steps = args.steps if is_head else max(args.steps, 100 if w.N <= 1024 else args.steps)
        entries[name] = measure(case, steps, args.warmup, flush_buf, 0.0 if is_head else args.warm_ms)
        if name == args.workload:
            head_case_x = case.x
        print(f"[bench] {name}: {entries[name]['tflops']} TFLOP/s, step {entries[name]['ms_per_step']} ms "
              f"({time.perf_counter() - t0:.1f} s)", file=sys.stderr, flush=True)
        del case
        torch.cuda.empty_cache()
    head = entries[args.workload]
    w = WORKLOADS[args.workload]
    result = {
        "metric": METRIC,
        "value": head["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAME[w.dtype],
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {WORKLOAD_TEXT[w.name]}", "global_batch": w.B, "heads": w.H,
                   "seq_len": w.N, "head_dim": w.d, "grad_dtype": "fp32", "parallelism": "none (1 GPU)"},
        "mfma_frac": head["mfma_frac"],
        "fwd_tflops": head["fwd_tflops"],
        "fwd_mfma_frac": head["fwd_mfma_frac"],
        "bwd_tflops": head.get("bwd_tflops"),
        "bwd_mfma_frac": head.get("bwd_mfma_frac"),
        "per_kernel": head["per_kernel"],
        "flushed": head["flushed"],
        "roofline": head["roofline"],
        "configs": [entries[n] for n in sorted(entries)],
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, head_case_x)
    print(json.dumps(result), flush=True)
    return 0


def run_roofs(args):
    """Microbenchmarks of the roofs the kernels are measured against (HIP
    kernels in the package's roofs library): MFMA rate and the clock it runs
    at, issue rates of the VALU instructions the kernels use, MFMA / VALU
    overlap, LDS read bandwidth (plain and transpose reads), the compute
    skeleton of a forward tile step, HBM copy and the empty-launch floor."""
    import torch

    from io_aware_exact_14_amd import roofs

    torch.cuda.set_device(0)
    out = roofs.run_all()
    out["device"] = torch.cuda.get_device_name(0)
    out["cus"] = torch.cuda.get_device_properties(0).multi_processor_count
    print(json.dumps(out), flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="C4", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--only", action="store_true", help="measure --workload alone (no configs array)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-flush", action="store_true", help="skip the cache-flushed steps (profiling runs)")
    ap.add_argument("--warm-ms", type=float, default=150.0,
                    help="device time of untimed steps before timing each workload other than the headline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 512 MiB device copy first (reference kernel for HBM counters)")
    ap.add_argument("--standard", action="store_true", help="standard vs tiled attention on --workload")
    ap.add_argument("--sweep", action="store_true", help="sequence-length sweep of the tiled kernels")
    ap.add_argument("--roofs", action="store_true", help="MFMA / VALU / LDS / tile skeleton / HBM / launch microbenchmarks")
    ap.add_argument("--sweep-n", default="1024,2048,4096,8192,16384,32768,65536")
    ap.add_argument("--sweep-d", default="64,128")
    ap.add_argument("--sweep-tokens", type=int, default=16384, help="B = max(1, tokens // N)")
    ap.add_argument("--standard-cap-gb", type=float, default=64.0)
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the attention path here is single-GPU "
              "(heads would shard over GPUs with no communication); run with --gpus 1", file=sys.stderr)
        return 2
    if args.roofs:
        return run_roofs(args)
    if args.standard:
        if args.workload == "C4" and "--workload" not in " ".join(sys.argv):
            args.workload = "C2"
        return run_standard(args)
    if args.sweep:
        return run_sweep(args)
    return run_main(args)


if __name__ == "__main__":
    sys.exit(main())
