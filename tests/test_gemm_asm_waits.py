"""Static check of where the GEMM K loops wait for their loads (CPU).

gemm.hip fills its LDS stage buffers by LDS-DMA and waits for a stage's
loads once per stage, at the barrier between the two halves of the stage;
the loads of the stage after next are issued while the other buffer is read.
That wait is written out (s_waitcnt vmcnt(0) before the barrier): the
compiler inserts one by itself only where its alias analysis cannot separate
an LDS read from the loads in flight, so relying on it would leave the
barrier unguarded whenever a schedule change lets it prove the reads apart
(a change of the MX kernels' scale handling once did exactly that).  The
first test checks, on every gemm_kernel and gemm_nvfp4_kernel
instantiation, that each barrier of the K loop follows a vmcnt(0) with no
load in between.
The compiler inserts its own vmcnt wait before any LDS read that it cannot
prove apart from an LDS-DMA load still in flight, and such a wait in the
middle of the loop costs the loads their lead (on the BF16 Dgrad / Wgrad
kernels, whose transposing reads carried no alias information, it made them
12-19% slower than with the lead).  The second test checks, for every
bf16-output instantiation
whose K loop is one machine loop, that the loop waits for loads only with
vmcnt(0) at its s_barrier and nowhere else; the three BF16 kernels (both
operands contraction-contiguous, one or both MN-contiguous) must be among
them.  Both compile the file for gfx950 with the library's own flags.
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


_LABEL = re.compile(r"^(\.LBB\w+:|; %bb\.\d+:)")


def loop_blocks(body):
    """[(header label, [block lines])] of the machine loops whose blocks hold
    matrix instructions: the header block and every block the compiler marks
    as inside that loop (a loop may span several blocks, not all after its
    header)."""
    blocks, cur = [], None
    for line in body:
        if _LABEL.match(line):
            cur = [line]
            blocks.append(cur)
        elif cur is not None:
            cur.append(line)
    out = []
    for blk in blocks:
        m = re.match(r"^\.L(BB\w+):.*Loop Header", blk[0])
        if not m:
            continue
        name = m.group(1)
        members = [b for b in blocks if b is blk or ("Header=" + name + " ") in b[0] + " "]
        if any(_op(l).startswith("v_mfma") for b in members for l in b):
            out.append((name, members))
    return out


def check_barrier_waits(block):
    """Violations of 'every s_barrier of this block follows a vmcnt(0) with no
    vector-memory load issued between the two' (a weaker vmcnt(N) wait in
    between, such as the compiler's own for the barrier, changes nothing)."""
    bad = []
    for i, line in enumerate(block):
        if _op(line) != "s_barrier":
            continue
        for prev in reversed(block[:i]):
            op = _op(prev)
            if op.startswith(("global_load", "buffer_load", "scratch_load", "flat_load")):
                bad.append(f"{prev.strip()!r} issued after the last vmcnt(0) before the barrier")
                break
            if op == "s_waitcnt" and "vmcnt(0)" in prev:
                break
        else:
            bad.append("a barrier with no vmcnt(0) before it in its block")
    return bad


def _salu(op):
    return op.startswith("s_") and op not in ("s_barrier", "s_endpgm") and not op.startswith(("s_cbranch", "s_branch"))


def check_loop_waits(loop):
    """Violations of 'the loop waits for loads only at its s_barrier': every
    vmcnt wait reaches the barrier through waits and scalar instructions only
    (the kernel's explicit vmcnt(0) and the compiler's own wait for the
    barrier may both be there, back to back), and one of them is vmcnt(0)."""
    bad = []
    waits = [(i, l) for i, l in enumerate(loop) if _op(l) == "s_waitcnt" and "vmcnt" in l]
    if not any("vmcnt(0)" in l for _, l in waits):
        return ["no vmcnt(0) wait in the K loop"]
    for i, l in waits:
        nxt = next((m for m in loop[i + 1:] if _op(m) and not _salu(_op(m))), "")
        if _op(nxt) != "s_barrier":
            bad.append(f"the K loop waits with {l.strip()!r} away from its barrier (next: {nxt.strip()!r})")
    return bad


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


def test_every_k_loop_barrier_follows_its_loads(asm_lines):
    fns = functions(asm_lines, "_ZN3pbs1[17]gemm_(?:nvfp4_)?kernel")
    assert len(fns) >= 28, sorted(fns)          # 24 gemm_kernel + 4 gemm_nvfp4_kernel
    for name, body in fns.items():
        loops = loop_blocks(body)
        assert loops, f"{name}: no K loop found"
        barriers = 0
        for _, members in loops:
            for blk in members:
                bad = check_barrier_waits(blk)
                assert not bad, f"{name}: " + "; ".join(bad)
                barriers += sum(1 for l in blk if _op(l) == "s_barrier")
        assert barriers >= 1, f"{name}: no barrier in the K loop"


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


def test_barrier_checker_catches_an_unguarded_barrier():
    """The barrier check itself: a barrier preceded only by lgkmcnt, by a
    counted vmcnt, or by a load after its vmcnt(0) is reported; the
    explicit-wait form passes, also with an lgkmcnt wait in between."""
    good = [".LBB0_1:", "\tglobal_load_lds_dwordx4 v0, s[0:1]", "\ts_waitcnt vmcnt(0)", "\ts_waitcnt lgkmcnt(0)",
            "\ts_barrier"]
    assert check_barrier_waits(good) == []
    assert check_barrier_waits([l.replace("vmcnt(0)", "lgkmcnt(0)") for l in good])
    assert check_barrier_waits([l.replace("vmcnt(0)", "vmcnt(4)") for l in good])
    late = good[:3] + ["\tglobal_load_lds_dwordx4 v1, s[0:1]"] + good[3:]
    assert check_barrier_waits(late)
    late_buf = good[:3] + ["\tbuffer_load_dwordx4 v1, s[4:7], s2 offen lds"] + good[3:]
    assert check_barrier_waits(late_buf)
    weaker_after = good[:3] + ["\ts_waitcnt vmcnt(2) lgkmcnt(0)"] + good[4:]
    assert check_barrier_waits(weaker_after) == []
    body = [".LBB0_2:                                ;   in Loop: Header=BB0_3 Depth=1", "\tv_mfma_x a[0:15]",
            ".LBB0_3:                                ; =>This Inner Loop Header: Depth=1"] + good[1:] + [
            "\ts_cbranch_scc0 .LBB0_2", ".LBB0_4:"]
    loops = loop_blocks(body)
    assert len(loops) == 1 and len(loops[0][1]) == 2


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
    both = head + ["\ts_waitcnt vmcnt(0)", "\ts_add_i32 s36, s38, s30", "\ts_waitcnt vmcnt(2) lgkmcnt(0)"] + good[3:]
    assert check_loop_waits(both) == []
