"""Compile the HIP sources into ``libmha.so`` (gfx950) next to this file.

Every call compiles from scratch (object files go to ``_build/``), one hipcc
process per translation unit, then links the shared library and swaps it in
atomically.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libmha.so")

SOURCES = ["api.hip", "gemm.hip", "attn_bf16.hip", "attn_f16.hip", "attn_f32.hip", "attn_merge.hip",
           "attn_bwd.hip"]

ARCH = "gfx950"
FLAGS = [
    "-O3", f"--offload-arch={ARCH}", "-fPIC", "-std=c++17", "-Wall",
    "-Wno-unused-function",
    # no packed fp32 arithmetic in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]
# Attention kernels: matrix-core results in ordinary VGPRs (no accumulator-
# register copies around the softmax arithmetic).  The GEMMs keep their
# accumulators wherever the compiler prefers (accumulation registers).
PER_SOURCE_FLAGS = {src: ["-mllvm", "-amdgpu-mfma-vgpr-form"]
                    for src in ("attn_bf16.hip", "attn_f16.hip", "attn_f32.hip", "attn_bwd.hip")}


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libmha.so")


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *FLAGS, *PER_SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src),
           "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    noise = "is not a recognized feature for this target"
    warn = "\n".join(l for l in res.stderr.splitlines() if noise not in l).strip()
    return obj, warn


def build(verbose=True):
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = []
    for obj, warn in results:
        objs.append(obj)
        if warn and verbose:
            print(warn, file=sys.stderr)
    tmp = LIB_PATH + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build()
