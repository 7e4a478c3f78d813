"""Python driver of libfa_roofs.so: microbenchmarks of the roofs the
attention kernels are measured against (bf16 MFMA rate and its clock,
issue rates of the VALU instructions the kernels use, MFMA / VALU overlap,
LDS read bandwidth, the compute skeleton of a forward tile step, HBM copy,
empty-launch floor).

Used by ``bench.py --roofs``. The library is built beside libfa.so by
``build.py``; it is measurement tooling, not part of the attention path.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_roofs.so")


def _load():
    if not os.path.exists(LIB_PATH):
        raise OSError(f"{LIB_PATH} is missing: build it with `python io_aware_exact_14_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    d = ctypes.POINTER(ctypes.c_double)
    lib.roofs_mfma.argtypes = [ctypes.c_int, ctypes.c_int, d, d, d]
    lib.roofs_valu.argtypes = [ctypes.c_int, ctypes.c_int, d, d, d]
    lib.roofs_lds.argtypes = [ctypes.c_int, ctypes.c_int, d, d, d]
    lib.roofs_overlap.argtypes = [ctypes.c_int, ctypes.c_int, d, d]
    lib.roofs_copy.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int, d, d]
    lib.roofs_launch.argtypes = [ctypes.c_int, ctypes.c_int, d]
    lib.roofs_skeleton.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, d, d]
    for f in (lib.roofs_mfma, lib.roofs_valu, lib.roofs_lds, lib.roofs_overlap, lib.roofs_copy, lib.roofs_launch,
              lib.roofs_skeleton):
        f.restype = ctypes.c_int
    return lib


def _d():
    return ctypes.c_double(0.0)


def run_all(cus: int | None = None) -> dict:
    """Runs every microbenchmark (one warm-up launch, then one timed launch
    each). Cycle counts use the clock each kernel itself ran at."""
    lib = _load()
    if cus is None:
        import torch

        cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = {"cus": cus}
    for label, iters in (("short", 20000), ("long", 200000)):
        tf, clk, ms = _d(), _d(), _d()
        rc = lib.roofs_mfma(iters, 2, ctypes.byref(tf), ctypes.byref(clk), ctypes.byref(ms))
        if rc != 0:
            raise RuntimeError(f"roofs_mfma failed ({rc})")
        out[f"mfma_bf16_tflops_{label}"] = round(tf.value, 2)
        out[f"mfma_clock_ghz_{label}"] = round(clk.value, 4)
        out[f"mfma_ms_{label}"] = round(ms.value, 3)
        # 32x32x16 bf16 MFMA: 32768 flops per wave instruction, 4 SIMDs per CU
        out[f"mfma_cycles_per_32x32x16_{label}"] = round(4 * cus * clk.value * 1e9 / (tf.value * 1e12 / 32768.0), 2)
    # kinds of rate_kernel; the last two issue two instructions per step
    kinds = (("exp", 0), ("fma", 1), ("dot2_bf16", 2), ("mul_lo_u32", 3), ("perm", 4), ("cvt_pk_bf16", 5),
             ("pk_mul_lo_u16", 6), ("exp4_fma4_mix", 9), ("cmp_cndmask_pair", 7), ("dpp_mov_add_pair", 8))
    for name, kind in kinds:
        r, clk, ms = _d(), _d(), _d()
        rc = lib.roofs_valu(kind, 20000, ctypes.byref(r), ctypes.byref(clk), ctypes.byref(ms))
        if rc != 0:
            raise RuntimeError(f"roofs_valu({name}) failed ({rc})")
        if kind in (0, 1):
            out[f"{name}_wave_inst_per_s"] = r.value
            out[f"{name}_clock_ghz"] = round(clk.value, 4)
            out[f"{name}_ms"] = round(ms.value, 3)
        out[f"{name}_cycles_per_wave_inst" if kind < 7 or kind == 9 else f"{name}_cycles_per_step"] = round(
            4 * cus * clk.value * 1e9 / r.value, 3)
    for nv in (0, 4, 8, 12, 16, 24):
        cyc, clk = _d(), _d()
        if lib.roofs_overlap(nv, 20000, ctypes.byref(cyc), ctypes.byref(clk)) != 0:
            raise RuntimeError("roofs_overlap failed")
        out[f"overlap_2mfma_{nv}fma_cycles"] = round(cyc.value, 2)
    for kind, name in ((0, "lds_read_b128"), (1, "lds_read_tr16_b64_pattern")):
        r, clk, ms = _d(), _d(), _d()
        if lib.roofs_lds(kind, 20000, ctypes.byref(r), ctypes.byref(clk), ctypes.byref(ms)) != 0:
            raise RuntimeError("roofs_lds failed")
        if kind == 0:
            out["lds_read_b128_tb_s"] = round(r.value / 1e12, 3)
            out["lds_clock_ghz"] = round(clk.value, 4)
            out["lds_ms"] = round(ms.value, 3)
        out[f"{name}_bytes_per_clk_per_cu"] = round(r.value / (cus * clk.value * 1e9), 1)
    for dh in (64, 128):
        for lds, pipe in ((0, 0), (1, 0)) + (((0, 1), (1, 1)) if dh == 128 else ()):
            cyc, clk = _d(), _d()
            if lib.roofs_skeleton(dh, lds, pipe, 4000, ctypes.byref(cyc), ctypes.byref(clk)) != 0:
                raise RuntimeError("roofs_skeleton failed")
            tag = f"skeleton_d{dh}_{'lds' if lds else 'regs'}{'_pipelined' if pipe else ''}"
            out[f"{tag}_cycles_per_tile"] = round(cyc.value, 1)
            # products per wave tile: 2 * d/16 (S) + 4 * d/32 (PV), 32 matrix-pipe cycles each
            out[f"{tag}_mfma_frac"] = round(32.0 * (2 * dh // 16 + 4 * dh // 32) / cyc.value, 3)
            out[f"{tag}_clock_ghz"] = round(clk.value, 4)
    best = None
    for bpc in (2, 8, 32):
        for unr in (1, 4, 8):
            r, ms = _d(), _d()
            if lib.roofs_copy(1 << 30, bpc, unr, ctypes.byref(r), ctypes.byref(ms)) != 0:
                raise RuntimeError("roofs_copy failed")
            out[f"hbm_copy_gb_s_wg{bpc}_unr{unr}"] = round(r.value / 1e9, 1)
            if best is None or r.value > best:
                best = r.value
    out["hbm_copy_gb_s_best"] = round(best / 1e9, 1)
    for blocks in (1, 4, 1024):
        us = _d()
        if lib.roofs_launch(blocks, 200, ctypes.byref(us)) != 0:
            raise RuntimeError("roofs_launch failed")
        out[f"empty_launch_us_{blocks}wg"] = round(us.value, 3)
    out["notes"] = ("MFMA: v_mfma_f32_32x32x16_bf16, 2 waves per SIMD x 4 independent chains, 20000 and 200000 "
                    "iterations. Clocks: s_memtime over s_memrealtime on wave 0 of each kernel. VALU kinds: 8 "
                    "independent chains per lane of one instruction, 4 waves per SIMD, cycles per wave "
                    "instruction per SIMD (pairs: per two-instruction step). Overlap: 2 independent MFMAs (64 "
                    "matrix-pipe cycles) plus n FMAs per iteration, SIMD cycles per wave iteration at 4 waves "
                    "per SIMD. LDS: ds_read_b128 of consecutive 16-byte chunks, and two ds_read_b64_tr_b16 per "
                    "lane in the kernels' transpose pattern (64-row bf16 tile, 144-byte rows), 4 waves per SIMD. Skeleton: a "
                    "forward tile step (32 queries x 64 keys per wave: S products, FMA + exp2 + bf16 pack + row "
                    "sum on 32 scores per lane, PV products) with no HBM traffic, K/V operands from registers or "
                    "from an LDS tile written once, 4 waves per SIMD at d=64 and 2 at d=128, plain or (d=128) software-"
                    "pipelined (the next step's S products issued between this step's exponentials, fenced, K "
                    "fragments read three products ahead); SIMD cycles per wave tile step and the matrix pipe's "
                    "share of them. HBM: 1 GiB device copy (read + write bytes counted), nontemporal "
                    "loads and stores, workgroups per CU x 16-byte elements per lane per step swept. Launch: 200 "
                    "back-to-back launches of an empty kernel (1, 4 or 1024 workgroups) between one event pair.")
    return out
