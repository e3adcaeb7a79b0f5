"""Build the CSA2 HIP library (libcsa2.so) in-tree for gfx950 with hipcc.

Usage: python -m compressed_sparse_attention_07_amd.build  (or build() from Python).
Each source is compiled to an object in _build/ (in parallel), then linked into
compressed_sparse_attention_07_amd/libcsa2.so next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcsa2.so")
SOURCES = ["fp4_pack.hip", "indexer.hip", "attend.hip", "attend_decode.hip", "noalloc.hip", "probe.hip",
           "csa2_api.cpp"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Per-source additions.  indexer.hip: MFMA results in ordinary VGPRs (no accumulation registers),
# so the scoring epilogues read them without a copy per value.
EXTRA = {"indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-kernarg-preload-count=16"],
         # all three: a kernel's leading scalar and pointer arguments preloaded into SGPRs at launch
         "attend.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=16"],
         "attend_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-kernarg-preload-count=16"],
         # fp4_pack.hip: the scale table is built by the compiler (constexpr), which needs more steps
         "fp4_pack.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=16", "-fconstexpr-steps=100000000"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(7, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
