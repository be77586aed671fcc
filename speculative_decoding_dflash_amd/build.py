"""Build libdflash.so (gfx950) in-tree with hipcc.

Usage: python -m speculative_decoding_dflash_amd.build   (or call build()).
Every HIP source is compiled for gfx950 only, with packed-fp32 instruction selection disabled; the
accept / resample stage is compiled without floating-point contraction so that its fp32 decisions
are reproducible exactly.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdflash.so")
BUILD = os.path.join(ROOT, "_build", "dflash")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument"]
SOURCES = {
    "gemm.hip": [],
    # accumulators of the MFMA loops in VGPRs: without this the 256-row tiles' loop body shuffled its
    # accumulators between AGPRs and VGPRs around every MFMA
    "gemm_tc.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "attention.hip": [],
    "rows.hip": [],
    "dflash2.hip": [],
    "sampler.hip": [],
    "decide.hip": ["-ffp-contract=off"],
    "api.cpp": ["-x", "hip"],
    "op_static.cpp": ["-x", "hip"],
}


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, "-c", os.path.join(CSRC, src), "-o", obj] + COMMON + list(extra)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-6000:]}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda kv: _compile(*kv), SOURCES.items()))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-6000:]}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
