"""Build ``liblora_mlp.so`` (the gfx950 HIP library) in-tree with hipcc.

Usage: ``python -m lora_swiglu_mlp_amd.build`` (or call :func:`build`).
The library lands next to this file; object files go to ``_build/``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblora_mlp.so")
SOURCES = ["gemm.hip", "gemm_bf16.hip", "skinny.hip", "rmsnorm.hip", "lora_mlp.cpp"]
ARCH = "gfx950"

# -packed-fp32-ops: never emit packed fp32 VALU ops (kept off on purpose).
HIPFLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # the ILP-first machine scheduler keeps the 256 MFMA accumulators of
            # the GEMM kernels in place (no AGPR<->VGPR shuffles in the K loop)
            "-mllvm", "-amdgpu-sched-strategy=iterative-ilp",
            "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if out.strip() and verbose:
        print(out)
    return out


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every source for gfx950 and link the shared library. Returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    flags = HIPFLAGS + list(extra_flags or [])
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = [] if src.endswith(".hip") else ["-x", "hip"]
        cmds.append([cc] + flags + lang + ["-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
