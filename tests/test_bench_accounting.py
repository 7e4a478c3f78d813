"""Host-side checks of the measurement arithmetic in bench.py.

The roofline figures bench.py reports are ratios of the work and bytes
below to measured kernel times, so the work model is pinned here against
values derived by hand from the workload shapes (GFLOP and MB to the digits
they are quoted with):

* forward flops 4*B*H*N^2*d, halved for causal; backward 2.5x the forward;
  block-sparse counts 4*B*H*d*128^2 per kept block;
* compulsory bytes: each tensor a kernel must read or write, once.
"""
from __future__ import annotations

import pytest

import bench
from workloads import C5_KEPT_BLOCKS, WORKLOADS

# (forward GFLOP, backward GFLOP) by the convention, worked out from the shapes.
CONVENTION_GFLOP = {
    "C1": (0.004194, 0.0),        # 4 * 128^2 * 64, forward only
    "C2": (17.18, 42.95),         # 4 * 8 * 16 * 1024^2 * 64 / 2
    "C3": (137.4, 343.6),         # 4 * 4 * 16 * 4096^2 * 64 / 2
    "C4": (2199.0, 5497.6),       # 4 * 1 * 32 * 16384^2 * 128 / 2
    "C5": (69.52, 173.8),         # 4 * 2 * 16 * 64 * 128^2 * 518
}


@pytest.mark.parametrize("name", sorted(CONVENTION_GFLOP))
def test_convention_flops(name):
    w = WORKLOADS[name]
    kept = C5_KEPT_BLOCKS if w.block_sparse else 0
    fwd, bwd = bench.convention_flops(w, kept)
    ef, eb = CONVENTION_GFLOP[name]
    assert fwd / 1e9 == pytest.approx(ef, rel=2e-3)
    assert bwd / 1e9 == pytest.approx(eb, rel=2e-3)


def test_kernel_model_c2_bytes_and_flops():
    # C2: one [B][H][N][d] bf16 tensor is 8*16*1024*64*2 B = 16.78 MB; a row
    # statistic is 8*16*1024*4 B = 0.524 MB; fp32 gradients 33.55 MB each.
    w = WORKLOADS["C2"]
    m = bench.kernel_model(w, 0, 2, 4)
    t, r, g = 16.777216e6, 0.524288e6, 33.554432e6
    # forward: read Q, K, V; write O and LSE
    assert m["fwd_kernel"][1] == pytest.approx(4 * t + r)
    # dQ: read Q, K, V, O, dO, LSE; write dQ and D
    assert m["bwd_dq_kernel"][1] == pytest.approx(5 * t + 2 * r + g)
    # dK/dV: read Q, K, V, dO, LSE, D; write dK, dV (the 135 MB compulsory figure)
    assert m["bwd_dkdv_kernel"][1] == pytest.approx(4 * t + 2 * r + 2 * g)
    assert m["bwd_dkdv_kernel"][1] / 1e6 == pytest.approx(135.3, abs=0.1)
    # flops: 2*d per visible pair per product; 2, 3 and 4 products
    pairs = 8 * 16 * 1024 * 1024 / 2
    assert m["fwd_kernel"][0] == pytest.approx(2 * 2 * 64 * pairs)
    assert m["bwd_dq_kernel"][0] == pytest.approx(3 * 2 * 64 * pairs)
    assert m["bwd_dkdv_kernel"][0] == pytest.approx(4 * 2 * 64 * pairs)
    # the forward kernel's products are exactly the convention's forward
    assert m["fwd_kernel"][0] == pytest.approx(bench.convention_flops(w, 0)[0])


def test_kernel_model_block_sparse_counts_kept_blocks():
    w = WORKLOADS["C5"]
    m = bench.kernel_model(w, C5_KEPT_BLOCKS, 2, 4)
    pairs = 2 * 16 * 128 * 128 * C5_KEPT_BLOCKS
    assert m["fwd_kernel"][0] == pytest.approx(4 * 64 * pairs)
    assert m["bwd_dkdv_kernel"][0] == pytest.approx(8 * 64 * pairs)


def test_kernel_model_forward_only_workload():
    assert set(bench.kernel_model(WORKLOADS["C1"], 0, 4, 4)) == {"fwd_kernel"}


def test_traffic_is_tied_to_the_kernel_sources(monkeypatch, tmp_path):
    # a counter summary is used only while its recorded source digest matches
    (tmp_path / "profiles").mkdir()
    f = tmp_path / "profiles" / "bwd_dkdv_kernel__C2__traffic.txt"
    digest = bench.src_digest()
    f.write_text(f"src_sha256: {digest}\ntraffic_bytes_per_dispatch: 146779177\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "src_digest", lambda: digest)  # the sources themselves stay where they are
    assert bench.read_traffic("bwd_dkdv_kernel", "C2") == 146779177.0
    assert bench.read_traffic("bwd_dq_kernel", "C2") is None  # no summary
    f.write_text("src_sha256: " + "0" * 64 + "\ntraffic_bytes_per_dispatch: 146779177\n")
    assert bench.read_traffic("bwd_dkdv_kernel", "C2") is None  # stale summary


def test_roofline_picks_the_binding_roof_and_reports_the_ratio():
    # C4 dK/dV: 4.398 TFLOP of algorithmic work against 1.08 GB compulsory:
    # MFMA-bound; achieved = flops / time, frac = achieved / 2500
    w = WORKLOADS["C4"]
    m = bench.kernel_model(w, 0, 2, 4)
    r = bench._roofline(w, m, "bwd_dkdv_kernel", 4.0, 2500.0)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == pytest.approx(4.398046511104e12 / 4e-3 / 1e12, rel=1e-6)
    assert r["frac"] == pytest.approx(r["achieved"] / 2500.0, rel=1e-4)
    # C2 dK/dV: 135.3 MB in 50 us is above the MFMA time of its 34.4 GFLOP: HBM-bound
    w2 = WORKLOADS["C2"]
    r2 = bench._roofline(w2, bench.kernel_model(w2, 0, 2, 4), "bwd_dkdv_kernel", 0.05, 2500.0)
    assert r2["bound"] == "hbm" and r2["unit"] == "GB/s"
    assert r2["achieved"] == pytest.approx(135.3e6 / 50e-6 / 1e9, rel=2e-3)


def test_more_than_one_gpu_is_refused(capsys, monkeypatch):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    assert bench.main() == 2
    assert "one GPU" in capsys.readouterr().err
