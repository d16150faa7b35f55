"""Build libhta.so in-tree: hipcc for gfx950, one object per source, in parallel.

Usage: ``python -m speculative_decoding_verification_hybrid_amd._build``.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libhta.so")
SOURCES = ["hta_api.hip", "prefix_mfma.hip", "prefix_valu.hip", "tree.hip", "merge.hip",
           "accept.hip", "prefix_dot.hip",
           "window.hip", "tree_build.hip", "noalloc.hip"]
ARCH = "gfx950"

# -packed-fp32-ops: keep hipcc from forming packed fp32 instructions (the host
# pass warns that it does not know the feature; that is harmless).
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-source additions: the split-KV MFMA kernel wants MFMA results in VGPRs
# (its scores go straight into the softmax; its P.V accumulators are pinned to
# AGPRs by inline assembly).
FILE_FLAGS = {"prefix_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def flags_for(src: str) -> list:
    return CFLAGS + FILE_FLAGS.get(src, [])


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + flags_for(src) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libhta.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
