"""Build libprr.so for gfx950 with hipcc (in-tree; the library lands in lib/).

Usage: python -m block_sparse_attention_quest_amd.build [--verbose]

Every HIP translation unit is compiled with -Xclang -target-feature -Xclang -packed-fp32-ops (no
packed fp32 VALU ops).  select.hip and calib.hip, which must reproduce plain float64 arithmetic bit for bit, are also
compiled with -ffp-contract=off (no fused multiply-add).
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
BUILD = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libprr.so")
ARCH = "gfx950"

SOURCES = {
    "attn.hip": [],
    "select.hip": ["-ffp-contract=off"],
    "calib.hip": ["-ffp-contract=off"],
    "step.hip": [],
    "step_fp8.hip": [],
    "step_layer.hip": [],
    "step_layer_fp8.hip": [],
    "append.hip": [],
    "check.hip": [],
    "budget.cpp": ["-ffp-contract=off"],
    "prr_api.cpp": ["-x", "hip"],
}

COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-mcode-object-version=5",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libprr.so)")


def _compile(src: str, extra: list, verbose: bool) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in r.stderr.splitlines() if ln.strip() and noise not in ln]
    if msgs and verbose:
        print("\n".join(msgs), flush=True)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link lib/libprr.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda kv: _compile(kv[0], kv[1], verbose), SOURCES.items()))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-mcode-object-version=5", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose="--verbose" in sys.argv)
