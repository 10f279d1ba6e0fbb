"""Static check of the block-128 GEMM's hand-scheduled memory accesses (CPU).

gemm_blk.hip issues its scale-word loads and scale-ring LDS reads as inline
assembly and waits for them explicitly (s_waitcnt lgkmcnt(0) / vmcnt(12) or
vmcnt(0)), because the compiler would otherwise make them wait for every
tile load in flight.  The compiler does not know those instructions write
their destination registers later, so the generated code must not read,
copy or overwrite such a register before the wait that covers it.  This
test compiles the file for gfx950 with the library's own flags and checks
exactly that on the assembly of every instantiation.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from precision_block_scaled_amd import build as B

SRC = os.path.join(B.CSRC, "gemm_blk.hip")


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
    return bool(m) and int(m.group(1)) <= 12


def check_asm(lines):
    """Returns (number of inline-asm loads checked, list of violations)."""
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


def test_inline_asm_loads_are_waited_for_before_use():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "gemm_blk.s")
        cmd = [hipcc, *B.compile_flags(), *B.EXTRA_FLAGS.get("gemm_blk.hip", []), "--cuda-device-only", "-S",
               SRC, "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        lines = open(out).read().split("\n")
    checked, bad = check_asm(lines)
    assert checked >= 4 * 20, f"expected the inline-asm loads of all 4 instantiations, found {checked}"
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
