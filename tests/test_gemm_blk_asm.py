"""Static check of the block-128 GEMM's hand-counted waits (CPU).

gemm_blk.hip fills its LDS stage buffers and scale ring by LDS-DMA (9 loads
per lane and stage: 8 tile loads and one scale word) and waits for them
with explicit s_waitcnt: vmcnt(0) in the middle of each stage, and in the
prologue vmcnt(9) -- stage 0 landed, stage 1's loads still in flight.  The
counted wait is right only if the compiler emits exactly the kernel's own
loads before it and no spill traffic (scratch accesses also count), so it is
used only where the kernel does not spill.  This test compiles the file for
gfx950 with the library's own flags and checks, on the assembly of every
instantiation: no scratch; the K loop's vector-memory instructions are
exactly one stage's loads, after its one vmcnt(0); the prologue issues 18
loads before vmcnt(9); and no inline-assembly load result is touched before
a wait covers it (the file has none today; the check guards the pattern).
check_waits(body, counted=False) is the rule for a kernel that may spill:
vmcnt(0) only.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from precision_block_scaled_amd import build as B

SRC = os.path.join(B.CSRC, "gemm_blk.hip")
LOADS_PER_STAGE = {"global_load_lds_dwordx4": 8, "global_load_lds_dword": 1}


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {f"{m.group(1)}{i}" for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {tok} if m else set()


def _split(line):
    body = line.split(";")[0].strip()
    parts = body.split(None, 1)
    if not parts:
        return "", []
    return parts[0], [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []


def _covering_wait(kind, line):
    if kind == "lgkm":
        return "lgkmcnt(0)" in line
    m = re.search(r"vmcnt\((\d+)\)", line)
    return bool(m) and int(m.group(1)) == 0


def check_asm(lines):
    """Inline-assembly loads: returns (number checked, list of violations)."""
    checked, bad = 0, []
    for n, line in enumerate(lines):
        op, ops = _split(line)
        if op not in ("ds_read_b32", "ds_read_b128", "global_load_dword"):
            continue
        if n == 0 or not lines[n - 1].strip().startswith(";;#ASMSTART"):
            continue                      # compiler-issued: the compiler tracks it
        checked += 1
        dst = _regs(ops[0])
        kind = "lgkm" if op.startswith("ds_") else "vm"
        for m in range(n + 1, len(lines)):
            op2, ops2 = _split(lines[m])
            if op2 == "s_waitcnt":
                if _covering_wait(kind, lines[m]):
                    break
                continue
            if not op2 or op2.startswith("."):
                if lines[m].startswith(".Lfunc_end"):
                    bad.append(f"line {n + 1}: no covering wait before the end of the kernel")
                    break
                continue
            touched = set()
            for o in ops2:
                touched |= _regs(o)
            if touched & dst:
                bad.append(f"line {n + 1} {line.strip()!r}: register used at line {m + 1} {lines[m].strip()!r}")
                break
    return checked, bad


def _is_vmem(op):
    return op.startswith(("global_", "buffer_", "scratch_", "flat_"))


def kernels(lines):
    """{name: (instruction lines, scratch bytes)} of every gemm_blk_kernel instantiation
    (the compiler's '; ScratchSize:' note follows each function's code)."""
    out, order, cur = {}, [], None
    for line in lines:
        m = re.match(r"^(_ZN3pbs15gemm_blk_kernel\w+):", line)
        if m:
            cur = m.group(1)
            out[cur] = [[], None]
            order.append(cur)
            continue
        if cur is not None:
            out[cur][0].append(line)
            if line.strip().startswith("s_endpgm"):
                cur = None
        m = re.search(r"; ScratchSize: (\d+)", line)
        if m and order and out[order[-1]][1] is None:
            out[order[-1]][1] = int(m.group(1))
    return {k: (v[0], v[1]) for k, v in out.items()}


def _vmcnts(lines):
    out = []
    for i, l in enumerate(lines):
        m = re.search(r"s_waitcnt\s.*vmcnt\((\d+)\)", l)
        if m:
            out.append((i, int(m.group(1))))
    return out


def check_waits(body, counted):
    """Violations of the explicit vmcnt accounting in one kernel's assembly.

    counted: the kernel uses the prologue's vmcnt(9) (no spill allowed);
    otherwise every vmcnt wait must be vmcnt(0)."""
    bad = []
    loops = []                          # (header index, back-edge index) of loops with matrix instructions
    for h, l in enumerate(body):
        if "Inner Loop Header" not in l:
            continue
        label = l.split(":")[0]
        back = [i for i, m in enumerate(body) if i > h and _split(m)[0].startswith("s_cbranch") and label in m]
        if back and any(_split(m)[0].startswith("v_mfma") for m in body[h:back[-1]]):
            loops.append((h, back[-1]))
    if len(loops) != 1:
        return [f"expected one K loop, found {len(loops)}"]
    head, back = loops[0]
    loop = body[head:back + 1]
    if not counted:
        nz = [c for _, c in _vmcnts(body) if c != 0]
        if nz:
            bad.append(f"vmcnt waits {nz} other than vmcnt(0) in a kernel that may spill")
        return bad
    counts, first_load = {}, None
    for i, l in enumerate(loop):
        op, _ = _split(l)
        if _is_vmem(op):
            counts[op] = counts.get(op, 0) + 1
            first_load = i if first_load is None else first_load
    waits = _vmcnts(loop)
    if counts != LOADS_PER_STAGE:
        bad.append(f"K loop vector-memory instructions {counts}, expected {LOADS_PER_STAGE}")
    if [c for _, c in waits] != [0]:
        bad.append(f"K loop vmcnt waits {[c for _, c in waits]}, expected one vmcnt(0)")
    elif first_load is not None and first_load < waits[0][0]:
        bad.append("a load of the K loop comes before its vmcnt(0)")
    pro = body[:head]
    w9 = [i for i, c in _vmcnts(pro) if c == 9]
    if len(w9) != 1:
        bad.append(f"expected one vmcnt(9) in the prologue, found {len(w9)}")
    else:
        n = sum(1 for l in pro[:w9[0]] if _is_vmem(_split(l)[0]))
        if n != 2 * sum(LOADS_PER_STAGE.values()):
            bad.append(f"{n} vector-memory instructions before the prologue's vmcnt(9), expected 18")
    others = [c for _, c in _vmcnts(body) if c not in (0, 9)]
    if others:
        bad.append(f"unexpected vmcnt waits {others}")
    return bad


def _compile():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "gemm_blk.s")
        cmd = [hipcc, *B.compile_flags(), *B.EXTRA_FLAGS.get("gemm_blk.hip", []), "--cuda-device-only", "-S",
               SRC, "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return open(out).read().split("\n")


@pytest.fixture(scope="module")
def asm_lines():
    return _compile()


def test_counted_waits_match_the_loads(asm_lines):
    ks = kernels(asm_lines)
    assert len(ks) == 6, sorted(ks)
    for name, (body, scratch) in ks.items():
        assert scratch == 0, f"{name}: {scratch} bytes of scratch; its counted wait needs none"
        bad = check_waits(body, True)
        assert not bad, f"{name}: " + "; ".join(bad)


def test_inline_asm_loads_are_waited_for_before_use(asm_lines):
    checked, bad = check_asm(asm_lines)
    assert not bad, "\n".join(bad[:10])


def test_checker_catches_an_early_use():
    """The checker itself: a register read before its wait is reported."""
    lines = [
        ";;#ASMSTART",
        "\tds_read_b128 v[10:13], v2 offset:0",
        ";;#ASMEND",
        "\tv_mov_b32_e32 v20, v11",
        "\ts_waitcnt lgkmcnt(0)",
    ]
    checked, bad = check_asm(lines)
    assert checked == 1 and len(bad) == 1
    ok = [lines[0], lines[1], lines[2], "\ts_waitcnt lgkmcnt(0)", "\tv_mov_b32_e32 v20, v11"]
    assert check_asm(ok) == (1, [])


def test_wait_checker_catches_miscounts():
    """The wait check itself: a stray vector-memory instruction, a load before
    the loop's wait, or a counted wait in a kernel that may spill is reported."""
    stage = ["\tglobal_load_lds_dwordx4 v0, s[0:1]"] * 8 + ["\tglobal_load_lds_dword v0, s[2:3]"]
    pro = stage * 2 + ["\ts_waitcnt vmcnt(9)"]
    loop_head = [".LBB0_1:   ; =>This Inner Loop Header: Depth=1", "\tv_mfma_x v[0:15]"]
    good = pro + loop_head + ["\ts_waitcnt vmcnt(0)"] + stage + ["\ts_cbranch_scc0 .LBB0_1"]
    assert check_waits(good, True) == []
    extra = good[:-1] + ["\tscratch_load_dword v5, off, s0"] + good[-1:]
    assert check_waits(extra, True)
    early = pro + loop_head + stage[:1] + ["\ts_waitcnt vmcnt(0)"] + stage[1:] + ["\ts_cbranch_scc0 .LBB0_1"]
    assert check_waits(early, True)
    assert check_waits(good, False)                     # vmcnt(9) where spills may happen
    spill_ok = [l.replace("vmcnt(9)", "vmcnt(0)") for l in good]
    assert check_waits(spill_ok, False) == []
