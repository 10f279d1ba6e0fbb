"""Static check of where the GEMM K loops wait for their loads (CPU).

gemm.hip fills its LDS stage buffers by LDS-DMA and waits for a stage's
loads once per stage, at the barrier between the two halves of the stage;
the loads of the stage after next are issued while the other buffer is read.
The compiler inserts its own vmcnt wait before any LDS read that it cannot
prove apart from an LDS-DMA load still in flight, and such a wait in the
middle of the loop costs the loads their lead (on the BF16 Dgrad / Wgrad
kernels, whose transposing reads carried no alias information, it made them
12-19% slower than with the lead).  This test compiles the file for gfx950
with the library's own flags and checks, for every bf16-output instantiation
whose K loop is one machine loop, that the loop has exactly one vmcnt wait,
vmcnt(0), directly before its s_barrier; the three BF16 kernels (both
operands contraction-contiguous, one or both MN-contiguous) must be among
them.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from precision_block_scaled_amd import build as B

SRC = os.path.join(B.CSRC, "gemm.hip")
# gemm_kernel<OP, LDA, LDB, SC, AFMT, BFMT, OUT_BF16> for OP = BF16 and the
# three operand layouts, bf16 output
BF16_KERNELS = {
    "_ZN3pbs11gemm_kernelILi0ELi0ELi0ELi0ELi0ELi0ELb1EEEvNS_8GemmArgsE",
    "_ZN3pbs11gemm_kernelILi0ELi0ELi1ELi0ELi0ELi0ELb1EEEvNS_8GemmArgsE",
    "_ZN3pbs11gemm_kernelILi0ELi1ELi1ELi0ELi0ELi0ELb1EEEvNS_8GemmArgsE",
}


def _op(line):
    body = line.split(";")[0].strip()
    return body.split(None, 1)[0] if body else ""


def functions(lines, prefix):
    """{name: instruction lines} of every function whose symbol starts with prefix."""
    out, cur = {}, None
    for line in lines:
        m = re.match(r"^(" + prefix + r"\w*):", line)
        if m:
            cur = m.group(1)
            out[cur] = []
            continue
        if cur is not None:
            out[cur].append(line)
            if line.strip().startswith("s_endpgm"):
                cur = None
    return out


def mfma_loops(body):
    """[(header, back edge)] of the machine loops that contain matrix instructions."""
    loops = []
    for h, l in enumerate(body):
        if "Loop Header" not in l:
            continue
        label = l.split(":")[0]
        back = [i for i, m in enumerate(body) if i > h and _op(m).startswith("s_cbranch") and label in m]
        if back and any(_op(m).startswith("v_mfma") for m in body[h:back[-1]]):
            loops.append((h, back[-1]))
    return loops


def check_loop_waits(loop):
    """Violations of 'one vmcnt(0), directly before the loop's s_barrier'."""
    waits = [(i, l) for i, l in enumerate(loop) if _op(l) == "s_waitcnt" and "vmcnt" in l]
    if len(waits) != 1:
        return [f"{len(waits)} vmcnt waits in the K loop: {[l.strip() for _, l in waits]}"]
    i, l = waits[0]
    if "vmcnt(0)" not in l:
        return [f"the K loop's wait is {l.strip()!r}, not vmcnt(0)"]
    nxt = next((m for m in loop[i + 1:] if _op(m)), "")
    if _op(nxt) != "s_barrier":
        return [f"the K loop's vmcnt(0) is followed by {nxt.strip()!r}, not its s_barrier"]
    return []


@pytest.fixture(scope="module")
def asm_lines():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "gemm.s")
        cmd = [hipcc, *B.compile_flags(), *B.EXTRA_FLAGS.get("gemm.hip", []), "--cuda-device-only", "-S", SRC,
               "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return open(out).read().split("\n")


def test_k_loops_wait_once_per_stage(asm_lines):
    fns = functions(asm_lines, "_ZN3pbs11gemm_kernel")
    checked = set()
    for name, body in fns.items():
        if not name.endswith("Lb1EEEvNS_8GemmArgsE"):
            continue                                  # fp32 output: not on the timed path
        loops = mfma_loops(body)
        if len(loops) != 1:
            continue
        h, e = loops[0]
        bad = check_loop_waits(body[h:e + 1])
        assert not bad, f"{name}: " + "; ".join(bad)
        checked.add(name)
    assert BF16_KERNELS <= checked, sorted(BF16_KERNELS - checked)


def test_checker_catches_a_wait_before_the_barrier_phase():
    """The check itself: an extra wait in the loop, or a wait that is not the
    barrier's, is reported."""
    head = [".LBB0_1:   ; =>This Inner Loop Header: Depth=1", "\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]"]
    good = head + ["\ts_waitcnt vmcnt(0) lgkmcnt(0)", "\ts_barrier", "\tglobal_load_lds_dwordx4 v0, s[0:1]",
                   "\tds_read_b64_tr_b16 v[8:9], v2", "\ts_cbranch_scc0 .LBB0_1"]
    assert mfma_loops(good) == [(0, len(good) - 1)]
    assert check_loop_waits(good) == []
    early = head + ["\ts_waitcnt vmcnt(0)", "\tds_read_b64_tr_b16 v[8:9], v2"] + good[2:]
    assert check_loop_waits(early)
    counted = [l.replace("vmcnt(0)", "vmcnt(4)") for l in good]
    assert check_loop_waits(counted)
    no_barrier = [l for l in good if "s_barrier" not in l]
    assert check_loop_waits(no_barrier)
