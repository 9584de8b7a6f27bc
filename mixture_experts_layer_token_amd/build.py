"""Build the HIP library libmoe_mi355x.so in-tree for gfx950.

    python -m mixture_experts_layer_token_amd.build [-v]

Every .hip/.cpp under csrc/ is compiled with hipcc into _build/ (in parallel)
and linked into mixture_experts_layer_token_amd/libmoe_mi355x.so.  hipcc
cross-compiles, so this runs without a GPU.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe_mi355x.so")
ARCH = "gfx950"

SOURCES = ["route.hip", "route_screen.hip", "permute.hip", "fold.hip", "proxy.hip", "path.hip", "ffn_stream.hip",
           "ffn_gemm.hip", "layout.hip", "combine.hip", "probe.hip", "noalloc.hip", "moe_abi.cpp"]

# Packed fp32 instructions are switched off (-packed-fp32-ops); the host pass
# warns that it does not know the feature, which is harmless.
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the MoE library)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    lines = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln]
    if verbose and lines:
        print("\n".join(lines), flush=True)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source and link the shared library; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".", "_") + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([hipcc, *CFLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    jobs = jobs or min(len(cmds), max(1, (os.cpu_count() or 4) // 2), 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
