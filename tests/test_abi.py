"""The C-ABI library on the CPU: it loads, exports every entry point that
include/pbs.h declares, and rejects bad arguments with the documented status
before anything is enqueued (no GPU call is made by these tests)."""
import os
import re
import subprocess

import pytest

import precision_block_scaled_amd as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pbs.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pbs_[a-z0-9_]+)\s*\(", text)))


def test_library_built_and_loads():
    if not os.path.exists(P.lib_path):
        pytest.skip("libpbs.so not built (run __graft_entry__.build())")
    assert P.pbs_version() == 4


def test_every_declared_symbol_is_exported():
    if not os.path.exists(P.lib_path):
        pytest.skip("libpbs.so not built")
    names = declared_functions()
    assert len(names) >= 12
    out = subprocess.run(["nm", "-D", "--defined-only", P.lib_path], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (pbs_[a-z0-9_]+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    # the Python binding mirrors exactly the declared functions
    assert sorted(P.SIGNATURES) == names


def _expect(status, fn, *args):
    with pytest.raises(P.PBSError) as e:
        fn(*args)
    assert e.value.status == status, str(e.value)


FAKE = 1 << 40          # a non-null, 16-byte aligned address never dereferenced


def test_cast_validation_codes():
    if not os.path.exists(P.lib_path):
        pytest.skip("libpbs.so not built")
    c = P.pbs_cast
    # shape not a multiple of 16
    _expect(2, c, P.PBS_RECIPE_MXFP8, FAKE, 100, 64, P.PBS_FMT_E4M3, 1, 0, 0, 0, None, None, FAKE, FAKE,
            None, None, 0)
    # bad orientation mask
    _expect(1, c, P.PBS_RECIPE_MXFP8, FAKE, 64, 64, P.PBS_FMT_E4M3, 0, 0, 0, 0, None, None, FAKE, FAKE,
            None, None, 0)
    # wrong format for the recipe
    _expect(3, c, P.PBS_RECIPE_MXFP8, FAKE, 64, 64, P.PBS_FMT_E5M2, 1, 0, 0, 0, None, None, FAKE, FAKE,
            None, None, 0)
    # RHT only for NVFP4, only on the col copy
    _expect(3, c, P.PBS_RECIPE_MXFP8, FAKE, 64, 64, P.PBS_FMT_E4M3, 2, 0, P.PBS_FLAG_RHT16, 0, None, None,
            None, None, FAKE, FAKE, 0)
    _expect(3, c, P.PBS_RECIPE_NVFP4, FAKE, 64, 64, P.PBS_FMT_E2M1, 1, 0, P.PBS_FLAG_RHT16, 0, FAKE, None,
            FAKE, FAKE, None, None, 0)
    # block128 needs the blocked dim to be a multiple of 128
    _expect(2, c, P.PBS_RECIPE_FP8_BLOCK128, FAKE, 64, 96, P.PBS_FMT_E4M3, 1, 0, 0, 0, None, None, FAKE,
            FAKE, None, None, 0)
    # power-of-two sub-channel: blocked dims multiples of 128, E4M3 only, scale words 4-byte aligned
    _expect(2, c, P.PBS_RECIPE_FP8_BLOCK128_POW2, FAKE, 64, 96, P.PBS_FMT_E4M3, 1, 0, 0, 0, None, None, FAKE,
            FAKE, None, None, 0)
    _expect(3, c, P.PBS_RECIPE_FP8_BLOCK128_POW2, FAKE, 64, 128, P.PBS_FMT_E5M2, 1, 0, 0, 0, None, None, FAKE,
            FAKE, None, None, 0)
    _expect(1, c, P.PBS_RECIPE_FP8_BLOCK128_POW2, FAKE, 64, 128, P.PBS_FMT_E4M3, 1, 0, 0, 0, None, None, FAKE,
            FAKE + 2, None, None, 0)
    # 2D-block casts and two-copy casts with stochastic rounding: at most 65535 tiles of 128 rows (the
    # other two-copy casts walk their tiles in a persistent grid and pass validation at that height)
    _expect(2, c, P.PBS_RECIPE_FP8_BLOCK128, FAKE, 128 * 65536, 128, P.PBS_FMT_E4M3, 1, 1, 0, 0, None, None, FAKE,
            FAKE, None, None, 0)
    _expect(2, c, P.PBS_RECIPE_NVFP4, FAKE, 128 * 65536, 128, P.PBS_FMT_E2M1, 3, 0, P.PBS_FLAG_SR, 0, FAKE, None,
            FAKE, FAKE, FAKE, FAKE, 0)
    # per-tensor FP8 needs the scale
    _expect(1, c, P.PBS_RECIPE_FP8_CURRENT, FAKE, 64, 64, P.PBS_FMT_E4M3, 1, 0, 0, 0, None, None, FAKE,
            None, None, None, 0)
    # the BF16 recipe has no cast: unsupported, never a silent pass-through
    _expect(3, c, P.PBS_RECIPE_BF16, FAKE, 64, 64, P.PBS_FMT_BF16, 1, 0, 0, 0, None, None, FAKE, None,
            None, None, 0)
    # misaligned input
    _expect(1, c, P.PBS_RECIPE_MXFP8, FAKE + 2, 64, 64, P.PBS_FMT_E4M3, 1, 0, 0, 0, None, None, FAKE,
            FAKE, None, None, 0)
    # unknown recipe
    _expect(1, c, 17, FAKE, 64, 64, P.PBS_FMT_E4M3, 1, 0, 0, 0, None, None, FAKE, FAKE, None, None, 0)
    assert "unknown recipe" in P.pbs_last_error()


def test_gemm_validation_codes():
    if not os.path.exists(P.lib_path):
        pytest.skip("libpbs.so not built")
    g = P.pbs_gemm
    _expect(2, g, P.PBS_RECIPE_BF16, P.PBS_FPROP, 100, 64, 64, FAKE, P.PBS_FMT_BF16, None, None, FAKE,
            P.PBS_FMT_BF16, None, None, FAKE, P.PBS_FMT_F32, 0)
    _expect(2, g, P.PBS_RECIPE_MXFP8, P.PBS_FPROP, 64, 64, 96, FAKE, P.PBS_FMT_E4M3, FAKE, None, FAKE,
            P.PBS_FMT_E4M3, FAKE, None, FAKE, P.PBS_FMT_F32, 0)
    _expect(3, g, P.PBS_RECIPE_MXFP8, P.PBS_FPROP, 64, 64, 128, FAKE, P.PBS_FMT_E5M2, FAKE, None, FAKE,
            P.PBS_FMT_E4M3, FAKE, None, FAKE, P.PBS_FMT_F32, 0)
    _expect(3, g, P.PBS_RECIPE_NVFP4, P.PBS_FPROP, 64, 64, 128, FAKE, P.PBS_FMT_E4M3, FAKE, FAKE, FAKE,
            P.PBS_FMT_E4M3, FAKE, FAKE, FAKE, P.PBS_FMT_F32, 0)
    _expect(3, g, P.PBS_RECIPE_BF16, P.PBS_FPROP, 64, 64, 64, FAKE, P.PBS_FMT_BF16, None, None, FAKE,
            P.PBS_FMT_BF16, None, None, FAKE, P.PBS_FMT_E4M3, 0)
    _expect(1, g, P.PBS_RECIPE_FP8_CURRENT, P.PBS_FPROP, 64, 64, 128, FAKE, P.PBS_FMT_E4M3, None, None,
            FAKE, P.PBS_FMT_E4M3, None, None, FAKE, P.PBS_FMT_F32, 0)
    _expect(1, g, P.PBS_RECIPE_BF16, 7, 64, 64, 64, FAKE, P.PBS_FMT_BF16, None, None, FAKE,
            P.PBS_FMT_BF16, None, None, FAKE, P.PBS_FMT_F32, 0)
    # stored operand rows beyond 16 MiB (tiles address rows with 32-bit offsets) and dims beyond 2^30
    _expect(2, g, P.PBS_RECIPE_BF16, P.PBS_FPROP, 64, 64, (16 << 20) // 2 + 64, FAKE, P.PBS_FMT_BF16, None,
            None, FAKE, P.PBS_FMT_BF16, None, None, FAKE, P.PBS_FMT_F32, 0)
    _expect(2, g, P.PBS_RECIPE_FP8_CURRENT, P.PBS_FPROP, 64, 64, (16 << 20) + 128, FAKE, P.PBS_FMT_E4M3, None,
            FAKE, FAKE, P.PBS_FMT_E4M3, None, FAKE, FAKE, P.PBS_FMT_F32, 0)
    _expect(2, g, P.PBS_RECIPE_BF16, P.PBS_FPROP, (1 << 30) + 16, 64, 64, FAKE, P.PBS_FMT_BF16, None, None,
            FAKE, P.PBS_FMT_BF16, None, None, FAKE, P.PBS_FMT_F32, 0)
    # power-of-two sub-channel: 128x128 weight blocks need N % 128; scale words 4-byte aligned
    _expect(2, g, P.PBS_RECIPE_FP8_BLOCK128_POW2, P.PBS_FPROP, 64, 80, 128, FAKE, P.PBS_FMT_E4M3, FAKE, None,
            FAKE, P.PBS_FMT_E4M3, FAKE, None, FAKE, P.PBS_FMT_F32, 0)
    _expect(1, g, P.PBS_RECIPE_FP8_BLOCK128_POW2, P.PBS_WGRAD, 64, 80, 128, FAKE, P.PBS_FMT_E4M3, FAKE + 1,
            None, FAKE, P.PBS_FMT_E4M3, FAKE, None, FAKE, P.PBS_FMT_F32, 0)


def test_gemm_amax_validation_codes():
    if not os.path.exists(P.lib_path):
        pytest.skip("libpbs.so not built")
    g = P.pbs_gemm_amax
    # c_amax null or misaligned
    _expect(1, g, P.PBS_RECIPE_BF16, P.PBS_FPROP, 64, 64, 64, FAKE, P.PBS_FMT_BF16, None, None, FAKE,
            P.PBS_FMT_BF16, None, None, FAKE, P.PBS_FMT_F32, None, 0)
    _expect(1, g, P.PBS_RECIPE_BF16, P.PBS_FPROP, 64, 64, 64, FAKE, P.PBS_FMT_BF16, None, None, FAKE,
            P.PBS_FMT_BF16, None, None, FAKE, P.PBS_FMT_F32, FAKE + 2, 0)
    # otherwise pbs_gemm's checks, still before anything is enqueued
    _expect(2, g, P.PBS_RECIPE_BF16, P.PBS_FPROP, 100, 64, 64, FAKE, P.PBS_FMT_BF16, None, None, FAKE,
            P.PBS_FMT_BF16, None, None, FAKE, P.PBS_FMT_F32, FAKE, 0)
    _expect(3, g, P.PBS_RECIPE_MXFP8, P.PBS_FPROP, 64, 64, 128, FAKE, P.PBS_FMT_E5M2, FAKE, None, FAKE,
            P.PBS_FMT_E4M3, FAKE, None, FAKE, P.PBS_FMT_F32, FAKE, 0)


def test_scalar_entry_validation():
    if not os.path.exists(P.lib_path):
        pytest.skip("libpbs.so not built")
    _expect(1, P.pbs_amax, FAKE, 16, 16, 0, 0, None, 0)
    _expect(1, P.pbs_amax, FAKE, 16, 16, 4, 0, FAKE, 0)
    _expect(2, P.pbs_amax, FAKE, 24, 16, P.PBS_FLAG_RHT16, 0, FAKE, 0)
    _expect(1, P.pbs_scale_from_amax, None, 448.0, FAKE, FAKE, 0)
    _expect(1, P.pbs_scale_from_amax, FAKE, -1.0, FAKE, FAKE, 0)
    _expect(1, P.pbs_delayed_state_bytes, 0)
    assert P.pbs_delayed_state_bytes(16) == 16 + 64
    assert P.pbs_delayed_scale(0) is None


def test_quantized_bytes_accounting():
    if not os.path.exists(P.lib_path):
        pytest.skip("libpbs.so not built")
    n_rows, n_cols = 16, 4096
    codes, scales = P.pbs_quantized_bytes(P.PBS_RECIPE_NVFP4, n_rows, n_cols, 0)
    n = n_rows * n_cols
    assert (codes, scales) == (n // 2, n // 16)
    assert 8 * (codes + scales + 4) / n == 4.5 + 32 / n
    assert P.pbs_quantized_bytes(P.PBS_RECIPE_MXFP8, 128, 256, 0) == (128 * 256, 128 * 8)
    assert P.pbs_quantized_bytes(P.PBS_RECIPE_FP8_BLOCK128, 256, 256, 1) == (65536, 16)
    assert P.pbs_quantized_bytes(P.PBS_RECIPE_FP8_BLOCK128, 256, 256, 0) == (65536, 256 * 2 * 4)
    _expect(2, P.pbs_quantized_bytes, P.PBS_RECIPE_MXFP8, 16, 48, 0)
    # power-of-two sub-channel: one 4-byte word per block, like the fp32 scales
    assert P.pbs_quantized_bytes(P.PBS_RECIPE_FP8_BLOCK128_POW2, 256, 256, 1) == (65536, 16)
    assert P.pbs_quantized_bytes(P.PBS_RECIPE_FP8_BLOCK128_POW2, 256, 256, 0) == (65536, 256 * 2 * 4)
    # channel-wise FP8: one fp32 scale per row
    assert P.pbs_quantized_bytes(P.PBS_RECIPE_FP8_CHANNEL, 48, 80, 0) == (48 * 80, 48 * 4)
