"""Row casts at the edges of their work split, bit for bit against the oracle.

The 1D-block row cast hands each lane 8 consecutive values of the flat
tensor at a time, eight such units per lane and step, so a wave step covers
4,096 values; a block of 16, 32 or 128 values is 2, 4 or 16 neighbouring
lanes, and units past the end of the tensor load element 0 and store
nothing.  The shapes below (rows and columns multiples of 16, as the casts
require) put the end of the tensor inside a wave step and a workgroup: 256
units (half a wave step), 768 (one and a half), 3,840 (seven and a half wave
steps, not a whole workgroup's four), and a whole number of steps.  Every
1D recipe with a row copy runs on them: per-tensor E4M3 and E5M2 (the latter with the
fused amax of delayed scaling), MXFP8, 1x128, 1x128 with power-of-two
scales, NVFP4 and MXFP4 with and without stochastic rounding, and the
channel-wise row copy, whose units are 8 values of one row.
"""
import numpy as np
import pytest
import torch

import precision_block_scaled_amd as P
import workloads as W
from oracle import recipes as R
from oracle.formats import bf16_to_f32
from tests.gpu_util import first_mismatch, scalar_gpu, to_gpu_bf16, to_np_f32, to_np_u8

pytestmark = pytest.mark.gpu

SHAPES = [(16, 128), (16, 384), (48, 640), (16, 4096)]
SEED = 42


def _x(shape, k):
    return W.activations(*shape, seed=300 + k)


def _cast(recipe, fmt, x, flags=0, scale=None, amax_out=None, code_cols=None, scale_shape=None, sdtype=torch.uint8):
    rows, cols = x.shape
    codes = torch.empty((rows, code_cols or cols), dtype=torch.uint8, device="cuda")
    scales = torch.empty(scale_shape, dtype=sdtype, device="cuda") if scale_shape else None
    P.pbs_cast(recipe, to_gpu_bf16(x), rows, cols, fmt, P.PBS_ROW, 0, flags, SEED, scale, amax_out, codes, scales,
               None, None)
    torch.cuda.synchronize()
    return codes, scales


@pytest.mark.parametrize("shape", SHAPES)
def test_per_tensor_e4m3(shape):
    x = _x(shape, 1)
    s = np.float32(448.0 / 3.0)
    codes, _ = _cast(P.PBS_RECIPE_FP8_CURRENT, P.PBS_FMT_E4M3, x, scale=scalar_gpu(s))
    assert first_mismatch(to_np_u8(codes), R.cast_pertensor(x, s, "e4m3")) is None


@pytest.mark.parametrize("shape", SHAPES)
def test_per_tensor_e5m2_fused_amax(shape):
    x = _x(shape, 2)
    s = np.float32(2.0 ** 10 * 1.3)
    amax = torch.full((1,), -1.0, device="cuda")
    codes, _ = _cast(P.PBS_RECIPE_FP8_DELAYED, P.PBS_FMT_E5M2, x, scale=scalar_gpu(s), amax_out=amax)
    assert first_mismatch(to_np_u8(codes), R.cast_pertensor(x, s, "e5m2")) is None
    assert to_np_f32(amax)[0] == R.amax(x)


@pytest.mark.parametrize("shape", SHAPES)
def test_mxfp8(shape):
    x = _x(shape, 3)
    rows, cols = shape
    codes, e8 = _cast(P.PBS_RECIPE_MXFP8, P.PBS_FMT_E4M3, x, scale_shape=(rows, cols // 32))
    want_codes, want_e8 = R.quantize_mxfp8(x, "row")
    assert first_mismatch(to_np_u8(e8), want_e8) is None
    assert first_mismatch(to_np_u8(codes), want_codes) is None


@pytest.mark.parametrize("shape", SHAPES)
def test_block128(shape):
    x = _x(shape, 4)
    rows, cols = shape
    codes, s_inv = _cast(P.PBS_RECIPE_FP8_BLOCK128, P.PBS_FMT_E4M3, x, scale_shape=(rows, cols // 128),
                         sdtype=torch.float32)
    want_codes, want_s = R.quantize_block128(x, "row", False)
    assert first_mismatch(to_np_f32(s_inv).view(np.uint32), want_s.view(np.uint32)) is None
    assert first_mismatch(to_np_u8(codes), want_codes) is None


@pytest.mark.parametrize("shape", SHAPES)
def test_block128_pow2(shape):
    x = _x(shape, 5)
    rows, cols = shape
    codes, words = _cast(P.PBS_RECIPE_FP8_BLOCK128_POW2, P.PBS_FMT_E4M3, x, scale_shape=(rows, cols // 128),
                         sdtype=torch.int32)
    want_codes, want_e8 = R.quantize_block128_pow2(x, "row", False)
    got_words = words.cpu().numpy().view(np.uint32)
    assert first_mismatch(got_words, want_e8.astype(np.uint32) * np.uint32(0x01010101)) is None
    assert first_mismatch(to_np_u8(codes), want_codes) is None


@pytest.mark.parametrize("sr", [False, True])
@pytest.mark.parametrize("shape", SHAPES)
def test_nvfp4(shape, sr):
    x = _x(shape, 6)
    rows, cols = shape
    S = R.nvfp4_tensor_scales(R.amax(x))[0]
    codes, d = _cast(P.PBS_RECIPE_NVFP4, P.PBS_FMT_E2M1, x, flags=P.PBS_FLAG_SR if sr else 0, scale=scalar_gpu(S),
                     code_cols=cols // 2, scale_shape=(rows, cols // 16))
    rnd = R.sr_random_for(x.shape, "row", SEED) if sr else None
    want_codes, want_d = R.quantize_nvfp4(bf16_to_f32(x), np.float32(S), sr_random=rnd)
    assert first_mismatch(to_np_u8(d), want_d) is None
    assert first_mismatch(to_np_u8(codes), want_codes) is None


@pytest.mark.parametrize("sr", [False, True])
@pytest.mark.parametrize("shape", SHAPES)
def test_mxfp4(shape, sr):
    x = _x(shape, 7)
    rows, cols = shape
    codes, e8 = _cast(P.PBS_RECIPE_MXFP4, P.PBS_FMT_E2M1, x, flags=P.PBS_FLAG_SR if sr else 0,
                      code_cols=cols // 2, scale_shape=(rows, cols // 32))
    rnd = R.sr_random_for(x.shape, "row", SEED) if sr else None
    want_codes, want_e8 = R.quantize_mxfp4(bf16_to_f32(x), sr_random=rnd)
    assert first_mismatch(to_np_u8(e8), want_e8) is None
    assert first_mismatch(to_np_u8(codes), want_codes) is None


@pytest.mark.parametrize("shape", SHAPES + [(16, 16), (32, 48)])
def test_channel_row(shape):
    x = _x(shape, 8)
    rows, _ = shape
    codes, s_inv = _cast(P.PBS_RECIPE_FP8_CHANNEL, P.PBS_FMT_E4M3, x, scale_shape=(rows,), sdtype=torch.float32)
    want_codes, want_s = R.quantize_channel(x, "row")
    assert first_mismatch(to_np_f32(s_inv).view(np.uint32), np.asarray(want_s, np.float32).view(np.uint32)) is None
    assert first_mismatch(to_np_u8(codes), want_codes) is None
