"""Build the gfx950 shared library libflashprefill.so in-tree.

    python -m block_sparse_long_kpool_amd.build

Each HIP translation unit is compiled separately (in parallel) with hipcc for
gfx950, then linked into block_sparse_long_kpool_amd/lib/libflashprefill.so.
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
BUILD = os.path.join(ROOT, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libflashprefill.so")
ARCH = "gfx950"

SOURCES = ["fp_api.hip", "fp_pool.hip", "fp_scores.hip", "fp_select.hip", "fp_attn.hip"]

# Packed fp32 VALU forms are disabled for all device code.  Device code runs
# with IEEE mode off (max / min then need no NaN canonicalisation; no kernel
# relies on NaN propagation: masked logits are -inf, never NaN).  Host code
# keeps full NaN semantics (argument validation tests for NaN).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-Xarch_device", "-mno-amdgpu-ieee", "-Xarch_device", "-fno-honor-nans"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _compile(src: str, extra: list) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-c",
           os.path.join(CSRC, src), "-o", obj, "-I", os.path.join(ROOT, "include"),
           "-Wno-unused-result"] + DEVICE_FLAGS + extra
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    return obj


def build(verbose: bool = True, extra: list | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    extra = list(extra or [])
    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
