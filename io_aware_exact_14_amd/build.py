"""Builds libfa.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python io_aware_exact_14_amd/build.py [--verbose] [--resource-usage]

It never imports the package (whose import loads the library).

Every .hip file under csrc/ is compiled to an object with hipcc, in
parallel, then linked into io_aware_exact_14_amd/libfa.so. The roofline
microbenchmarks under roofs/ are built the same way into a library of their
own, io_aware_exact_14_amd/libfa_roofs.so (measurement tooling for
``bench.py --roofs``; the attention path never loads it). Packed fp32 VALU
instructions are disabled for all device code.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")
ROOFS_SRC = os.path.join(PKG, "roofs")
ROOFS_LIB = os.path.join(PKG, "libfa_roofs.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libfa)")


def _flags(resource_usage: bool):
    f = [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{INCLUDE}",
        f"-I{CSRC}",
        "-Wall",
        "-Wno-unused-function",
    ]
    if resource_usage:
        f.append("-Rpass-analysis=kernel-resource-usage")
    return f


def _build_lib(cc, srcs, out, flags, verbose, jobs):
    def compile_one(src):
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        cmd = [cc, *flags, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        return src, obj, r

    objs = []
    with cf.ThreadPoolExecutor(jobs) as ex:
        for src, obj, r in ex.map(compile_one, srcs):
            if verbose or r.returncode != 0:
                msg = (r.stdout + r.stderr).strip()
                msg = "\n".join(l for l in msg.splitlines() if "packed-fp32-ops" not in l)
                if msg:
                    print(f"== {os.path.basename(src)}\n{msg}", file=sys.stderr)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}")
            objs.append(obj)
    tmp = out + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False, resource_usage: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    flags = _flags(resource_usage)
    jobs = jobs or min(len(srcs) + 1, max(1, (os.cpu_count() or 4)))
    _build_lib(cc, srcs, LIB, flags, verbose, jobs)
    roofs = sorted(glob.glob(os.path.join(ROOFS_SRC, "*.hip")))
    if roofs:
        _build_lib(cc, roofs, ROOFS_LIB, flags, verbose, jobs)
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true")
    args = ap.parse_args()
    print(build(args.verbose, args.resource_usage))


if __name__ == "__main__":
    main()
