"""Build libmoe.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m combine_top_router_amd.build   (or __graft_entry__.build()).
Every call recompiles every source.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
SOURCES = ["api.hip", "route.hip", "index.hip", "gemm.hip", "gemm_mx.hip", "gemm_fw.hip", "gemm_f32.hip", "mx_quant.hip",
           "router_gemm.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe)")


FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay off: plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# Kernels whose load waves stage operands in registers through inline-asm loads (jobs with
# REG = true).  The compiler sees such a load's destination as written at issue, so a
# spill in the kernel could copy, or a reuse overwrite, a register whose load is still in
# flight: these kernels must not spill at all.
REG_KERNELS = ("k_fwd_gateupILb0E", "k_fwd_downILb0E", "k_bwd_daILb0E", "k_bwd_dxILb0E")


def _check_no_spill(src: str, remarks: str) -> None:
    name = None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name and any(k in name for k in REG_KERNELS) and int(m.group(1)) > 0:
            raise RuntimeError(f"{src}: register-staged kernel {name} spills {m.group(1)} bytes per lane")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    extra = ["-Rpass-analysis=kernel-resource-usage"] if src == "gemm.hip" else []
    cmd = [hipcc(), *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-6000:]}")
    if extra:
        _check_no_spill(src, r.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-6000:]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
