"""Builds the gfx950 shared library libpa_gfx950.so in place (hipcc, no JIT cache)."""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpa_gfx950.so")
SOURCES = ["api.cpp", "stage1.hip", "merge.hip", "quant.hip", "gather.hip"]
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         # keep hipcc from emitting packed fp32 ops (v_pk_*_f32)
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # keep MFMA accumulators in VGPRs: the online-softmax rescale then multiplies
         # them in place instead of copying AGPR <-> VGPR every tile
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(jobs: int = 8, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(jobs=int(sys.argv[1]) if len(sys.argv) > 1 else 8)
