"""No silent fallback, observed the way the pages suggest ("How to optimize
Transformer-based models for low-precision training", "Interpreting results
for a real model": turn the dispatch log on and confirm that the low-precision
kernels actually run): with PBS_LOG_LEVEL=1 every recipe's Fprop GEMM and
casts log the kernel family of that recipe, in a child process so that the
environment variable is read at start-up."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import sys, torch
sys.path.insert(0, sys.argv[1])
import workloads as W
import precision_block_scaled_amd as P
from precision_block_scaled_amd import pipeline as PL
from tests.gpu_util import to_gpu_bf16
x, w = W.tiny_current_case(0)
dy = W.grads(256, 256, seed=3)
xg, wg, dyg = to_gpu_bf16(x), to_gpu_bf16(w), to_gpu_bf16(dy)
for r in sys.argv[2].split(","):
    states = None
    if r == "fp8_delayed":
        states = {k: PL.DelayedState(P.PBS_FMT_E5M2 if k == "dy" else P.PBS_FMT_E4M3, "cuda") for k in ("x", "w", "dy")}
    print(f"[recipe] {r}", file=sys.stderr, flush=True)
    A, B = PL.quantize_pass(r, "fprop", xg, wg, dyg, states=states)
    PL.gemm(r, "fprop", A, B, 256, 256, 512)
    torch.cuda.synchronize()
    sys.stderr.flush()
"""

EXPECT = {  # recipe -> (GEMM family, cast family or None)
    "bf16": ("gemm_bf16", None),
    "fp8_current": ("gemm_fp8_tensor", "cast_tensor_fp8"),
    "fp8_delayed": ("gemm_fp8_tensor", "cast_tensor_fp8"),
    "fp8_block128": ("gemm_fp8_block128", "cast_block128"),
    "mxfp8": ("gemm_mxfp8", "cast_mxfp8"),
    "nvfp4": ("gemm_nvfp4", "cast_nvfp4"),
    "mxfp4": ("gemm_mxfp4", "cast_mxfp4"),
    "fp8_channel": ("gemm_fp8_channel", None),
    "fp8_block128_1d1d": ("gemm_fp8_block128_1d1d", "cast_block128"),
    "fp8_block128_2d2d": ("gemm_fp8_block128_2d2d", "cast_block128"),
    "fp8_block128_pow2": ("gemm_fp8_block128_pow2", "cast_block128_pow2"),
}


def test_dispatch_log_names_each_recipes_kernels():
    env = dict(os.environ, PBS_LOG_LEVEL="1")
    r = subprocess.run([sys.executable, "-c", SCRIPT, ROOT, ",".join(EXPECT)], capture_output=True, text=True,
                       env=env, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    sections = {}
    cur = None
    for line in r.stderr.splitlines():
        if line.startswith("[recipe] "):
            cur = line.split()[1]
            sections[cur] = []
        elif line.startswith("[pbs] ") and cur:
            sections[cur].append(line)
    for rec, (gemm, cast) in EXPECT.items():
        lines = sections.get(rec, [])
        gemm_lines = [l for l in lines if " layout=" in l]
        # exactly one GEMM, of this recipe's family (no fallback to another format)
        assert len(gemm_lines) == 1 and gemm_lines[0].startswith("[pbs] " + gemm + " "), (rec, lines)
        if cast:
            assert any(l.startswith("[pbs] " + cast + "_") or l.startswith("[pbs] " + cast + " ")
                       for l in lines), (rec, lines)
