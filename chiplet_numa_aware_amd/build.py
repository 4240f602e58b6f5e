"""Builds libattn_numa.so (the HIP kernels and the C ABI) in-tree for gfx950.

Usage: python -m chiplet_numa_aware_amd.build  (or build() from Python).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libattn_numa.so")
SOURCES = [os.path.join(CSRC, name) for name in (
    "attn_fwd_d128.hip", "attn_fwd_d64.hip", "attn_bwd.hip", "attn_decode.hip", "attn_fwd.hip",
    "attn_numa.hip", "cac_gemm.hip")]
ARCH = os.environ.get("ATTN_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    # The kernels use +-inf but never produce or test NaN: lets max
    # reductions map to v_max3 without quieting every operand.
    "-fno-honor-nans",
    # No packed-fp32 VALU instructions anywhere in the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wall", "-Wno-unused-function",
]


def compile_command(src: str, obj: str) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", *FLAGS, "-c", src, "-o", obj]


def link_command(objs: list[str], out: str = LIB) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out]


def build(verbose: bool = False) -> str:
    """Compiles the library (always; the sources in parallel) and returns its path."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(src) + ".o") for src in SOURCES]
    procs = []
    for src, obj in zip(SOURCES, objs):
        cmd = compile_command(src, obj)
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                      text=True))
    failed = []
    for src, p in zip(SOURCES, procs):
        out, _ = p.communicate()
        if p.returncode != 0:
            sys.stderr.write(out)
            failed.append(os.path.basename(src))
    if failed:
        raise RuntimeError(f"hipcc failed on {', '.join(failed)}")
    tmp = LIB + ".tmp"
    cmd = link_command(objs, tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc link failed with exit code {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
