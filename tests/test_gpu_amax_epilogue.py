"""GPU checks of the per-tensor maximum: the amax kernel at ragged sizes with
the maximum planted at the ends and in the tail, and the GEMM epilogue's
max |C| (pbs_gemm_amax) against the exact maximum of the C it stores.

The maximum is exact (no rounding), so both must agree bit for bit with
NumPy's maximum of the same values; pbs_gemm_amax's C must equal
pbs_gemm's bit for bit.
"""
import numpy as np
import pytest
import torch

import workloads as W
import precision_block_scaled_amd as P
from precision_block_scaled_amd import pipeline as PL
from oracle import recipes as R
from oracle.formats import bf16_to_f32
from tests.gpu_util import to_gpu_bf16, to_np_f32

pytestmark = pytest.mark.gpu


def _sync():
    torch.cuda.synchronize()


@pytest.mark.parametrize("shape", [(999, 1001), (1000, 1000), (4096, 1040), (3, 5)])
@pytest.mark.parametrize("where", ["first", "last", "middle"])
def test_amax_planted(shape, where):
    x = W.grads(*shape, seed=91) if shape[0] >= 16 else W.grads(16, 16, seed=91)[:shape[0], :shape[1]].copy()
    t = bf16_to_f32(x).copy()
    n = t.size
    idx = {"first": 0, "last": n - 1, "middle": n // 2 + 3}[where]
    t.reshape(-1)[idx] = -7.5e4                    # larger than every other value
    x = W.f32_to_bf16_bits(t)
    out = torch.full((1,), -1.0, device="cuda")
    P.pbs_amax(to_gpu_bf16(x), shape[0], shape[1], 0, 0, out)
    _sync()
    assert to_np_f32(out)[0] == R.amax(x) == np.float32(abs(bf16_to_f32(x).reshape(-1)[idx]))


RECIPES = ["bf16", "fp8_current", "fp8_block128", "fp8_block128_2d2d", "mxfp8", "nvfp4", "mxfp4",
           "fp8_channel", "fp8_block128_pow2"]


@pytest.mark.parametrize("recipe", RECIPES)
@pytest.mark.parametrize("pass_", ["fprop", "dgrad", "wgrad"])
def test_gemm_amax_matches_stored_output(recipe, pass_):
    # Dgrad's output columns are K_in: 272 leaves a ragged 256-tile where the
    # blocks allow it (128-blocks need K_in % 128; MXFP4 needs its
    # contraction N_out % 256)
    M_tok, K_in, N_out = 512, 272 if pass_ == "dgrad" else 256, 384
    if recipe in ("fp8_block128", "fp8_block128_2d2d", "fp8_block128_pow2"):
        K_in = 256
    if recipe == "mxfp4" and pass_ == "dgrad":
        N_out = 512
    x = W.activations(M_tok, K_in, seed=92)
    w = W.weights(N_out, K_in, seed=93)
    dy = W.grads(M_tok, N_out, seed=94)
    M, N, K = PL.pass_dims(pass_, M_tok, K_in, N_out)
    A, B = PL.quantize_pass(recipe, pass_, to_gpu_bf16(x), to_gpu_bf16(w), to_gpu_bf16(dy))
    for out_dtype in (torch.float32, torch.bfloat16):
        C1 = PL.gemm(recipe, pass_, A, B, M, N, K, out_dtype=out_dtype)
        amax = torch.full((1,), -1.0, device="cuda")
        C2 = PL.gemm(recipe, pass_, A, B, M, N, K, out_dtype=out_dtype, c_amax=amax)
        _sync()
        assert torch.equal(C1.view(torch.int16) if out_dtype == torch.bfloat16 else C1.view(torch.int32),
                           C2.view(torch.int16) if out_dtype == torch.bfloat16 else C2.view(torch.int32))
        want = np.float32(np.abs(C2.float().cpu().numpy()).max())
        assert to_np_f32(amax)[0] == want, (out_dtype, to_np_f32(amax)[0], want)
        if out_dtype == torch.bfloat16:            # the same value pbs_amax reads from C
            a2 = torch.zeros(1, device="cuda")
            P.pbs_amax(C2, M, N, 0, 0, a2)
            _sync()
            assert to_np_f32(a2)[0] == want


def test_gemm_amax_empty_and_errors():
    C = torch.empty((0, 16), dtype=torch.float32, device="cuda")
    amax = torch.full((1,), 5.0, device="cuda")
    P.pbs_gemm_amax(P.PBS_RECIPE_BF16, P.PBS_FPROP, 0, 16, 64, C, P.PBS_FMT_BF16, None, None, C, P.PBS_FMT_BF16,
                    None, None, C, P.PBS_FMT_F32, amax)
    _sync()
    assert to_np_f32(amax)[0] == 0.0
    C = torch.full((32, 16), 3.0, dtype=torch.float32, device="cuda")
    amax.fill_(5.0)
    A = torch.zeros((32, 64), dtype=torch.bfloat16, device="cuda")
    P.pbs_gemm_amax(P.PBS_RECIPE_BF16, P.PBS_FPROP, 32, 16, 0, A, P.PBS_FMT_BF16, None, None, A, P.PBS_FMT_BF16,
                    None, None, C, P.PBS_FMT_F32, amax)
    _sync()
    assert to_np_f32(amax)[0] == 0.0 and float(C.abs().max()) == 0.0
    with pytest.raises(P.PBSError):
        P.pbs_gemm_amax(P.PBS_RECIPE_BF16, P.PBS_FPROP, 32, 16, 64, A, P.PBS_FMT_BF16, None, None, A,
                        P.PBS_FMT_BF16, None, None, C, P.PBS_FMT_F32, None)


@pytest.mark.parametrize("orient", ["row", "col"])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fused_amax_cast_more_tiles_than_workgroups(orient, fmt):
    """The per-tensor cast with its amax fused (delayed scaling) on a ragged
    tensor large enough that each of its at most 1024 workgroups walks
    several tiles (col copy) or segments (row copy): codes as the oracle's
    cast with the same scale, amax exact."""
    rows, cols = 2064, 8272                         # 9 x 130 col tiles, ragged in both
    x = W.grads(rows, cols, seed=95) if fmt == "e5m2" else W.activations(rows, cols, seed=95)
    s = np.float32(448.0 if fmt == "e4m3" else 57344.0) / R.amax(x) * np.float32(0.75)
    scale = torch.tensor([s], dtype=torch.float32, device="cuda")
    amax = torch.full((1,), -1.0, device="cuda")
    out = torch.empty((rows, cols) if orient == "row" else (cols, rows), dtype=torch.uint8, device="cuda")
    pfmt = P.PBS_FMT_E4M3 if fmt == "e4m3" else P.PBS_FMT_E5M2
    rc, cc = (out, None) if orient == "row" else (None, out)
    P.pbs_cast(P.PBS_RECIPE_FP8_DELAYED, to_gpu_bf16(x), rows, cols, pfmt, P.PBS_ROW if orient == "row" else P.PBS_COL,
               0, 0, 0, scale, amax, rc, None, cc, None)
    _sync()
    want = R.cast_pertensor(x, np.float32(s), fmt, orient)
    got = out.cpu().numpy()
    bad = np.argwhere(got != want)
    assert len(bad) == 0, f"{len(bad)} codes differ, first at {tuple(bad[0])}"
    assert to_np_f32(amax)[0] == R.amax(x)


@pytest.mark.parametrize("recipe", ["fp8_current", "nvfp4"])
def test_gemm_output_quantized_with_epilogue_amax(recipe):
    """Y = X W^T with its max |Y| from the epilogue, then Y quantized with
    current scaling (FP8) or NVFP4's tensor scale from that value and no amax
    pass: the codes and scales are the oracle's quantization of the stored Y."""
    from oracle.passes import quantize_operand
    x = W.activations(512, 256, seed=96)
    w = W.weights(384, 256, seed=97)
    dy = W.grads(512, 384, seed=98)
    A, B = PL.quantize_pass("fp8_current", "fprop", to_gpu_bf16(x), to_gpu_bf16(w), to_gpu_bf16(dy))
    amax = torch.zeros(1, device="cuda")
    Y = PL.gemm("fp8_current", "fprop", A, B, 512, 384, 256, out_dtype=torch.bfloat16, c_amax=amax)
    q = PL.quantize(recipe, Y, "x", "row", "fprop", known_amax=amax)
    _sync()
    ybits = Y.view(torch.int16).cpu().numpy().view(np.uint16)
    want = quantize_operand(recipe, "x", "row", ybits, "fprop")
    assert (q.codes.cpu().numpy() == want.codes).all()
    if recipe == "nvfp4":
        assert (q.scales.cpu().numpy() == want.scale).all()
    assert q.tensor_scale_inv.cpu().numpy().view(np.uint32)[0] == np.float32(want.tensor_scale_inv).view(np.uint32)
