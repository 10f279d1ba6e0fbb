"""Build libpbs.so (the HIP kernels and their C ABI) for gfx950, in-tree.

Usage: python -m precision_block_scaled_amd.build [--jobs N]

Every source is compiled by hipcc for gfx950 only.  Flags:
  -O3 -std=c++17 -fPIC
  -ffp-contract=off      the scale and cast arithmetic is a fixed sequence of
                         single fp32 operations; no multiply-add fusion
  -Xclang -target-feature -Xclang -packed-fp32-ops
                         no packed-fp32 VALU instructions
  -mllvm -disable-promote-alloca-to-lds
                         keep private arrays in registers (the GEMM's LDS
                         budget is spoken for)
gemm_blk.hip adds -mllvm -amdgpu-mfma-vgpr-form=1: its MFMAs write their
partial products to VGPRs, where the vector unit folds them (the other GEMMs
keep 256 accumulators per lane in AGPRs and must not take it).
fp32 division stays IEEE correctly rounded (hipcc's default) and fp32
denormals are kept (no flush-to-zero), which the bit-exact casts rely on.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libpbs.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["api.hip", "amax.hip", "cast.hip", "gemm.hip", "gemm_blk.hip"]
EXTRA_FLAGS = {"gemm_blk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
ARCH = "gfx950"


def hipcc():
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return p


def compile_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
            "-fno-gpu-flush-denormals-to-zero",
            "-mllvm", "-disable-promote-alloca-to-lds",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(HERE, "..", "include")]


def build(jobs=None, verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    objs = []

    def one(src):
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        cmd = [cc, *compile_flags(), *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(jobs or min(8, len(SOURCES))) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.v))
    sys.exit(0)
