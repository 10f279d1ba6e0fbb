"""GPU parity for the 1D1D and 2D2D sub-channel FP8 pairings (1x128 blocks
on every tensor, or 128x128 blocks on every tensor) through the C ABI.

Casts must match the oracle bit for bit (codes and fp32 scales); GEMMs must
lie within the FP8 bound (|err| <= 1e-5 * sum_k |a_k b_k| plus the 8-wide
dot unit's term, + 1 bf16 ulp for bf16 outputs) of the fp64 product of the
oracle-dequantized operands.
"""
import numpy as np
import pytest
import torch

import workloads as W
import precision_block_scaled_amd as P
from precision_block_scaled_amd import pipeline as PL
from oracle import recipes as R
from oracle.gemm_ref import gemm_ref, check_gemm, fp8_dot_unit_bound
from oracle.passes import pass_operands, quantize_operand
from tests.gpu_util import to_gpu_bf16, to_np_u8, to_np_f32, out_to_np, first_mismatch

pytestmark = pytest.mark.gpu

PAIRINGS = ["fp8_block128_1d1d", "fp8_block128_2d2d"]
CAST_CASES = [  # (src, orient, pass): every copy the three GEMMs consume
    ("x", "row", "fprop"), ("w", "row", "fprop"), ("w", "col", "dgrad"), ("dy", "row", "dgrad"),
    ("x", "col", "wgrad"), ("dy", "col", "wgrad")]


def _sync():
    torch.cuda.synchronize()


@pytest.mark.parametrize("recipe", PAIRINGS)
@pytest.mark.parametrize("src,orient,pass_", CAST_CASES)
@pytest.mark.parametrize("shape", [(256, 384), (384, 128)])
def test_cast_pairing(recipe, src, orient, pass_, shape):
    gen = {"x": W.activations, "w": W.weights, "dy": W.grads}[src]
    x = gen(*shape, seed=71)
    q = PL.quantize(recipe, to_gpu_bf16(x), src, orient, pass_)
    _sync()
    want = quantize_operand(recipe, src, orient, x, pass_)
    assert q.weight_2d == want.weight_2d
    assert first_mismatch(to_np_f32(q.scales).view(np.uint32), want.scale.view(np.uint32)) is None
    assert first_mismatch(to_np_u8(q.codes), want.codes) is None


GEMM_DIMS = {  # (M, N, K)
    "fp8_block128_1d1d": [(256, 384, 512), (272, 400, 256), (256, 256, 1536), (528, 272, 2304)],
    "fp8_block128_2d2d": [(256, 384, 512), (384, 256, 128), (256, 256, 1536), (512, 384, 2304)],
}


def tensor_shapes(pass_, M, N, K):
    return {"fprop": (M, K, N), "dgrad": (M, N, K), "wgrad": (K, M, N)}[pass_]


@pytest.mark.parametrize("recipe,dims", [(r, d) for r in PAIRINGS for d in GEMM_DIMS[r]])
@pytest.mark.parametrize("pass_", ["fprop", "dgrad", "wgrad"])
def test_gemm_pairing_parity(recipe, dims, pass_):
    M_tok, K_in, N_out = tensor_shapes(pass_, *dims)
    x = W.activations(M_tok, K_in, seed=1)
    w = W.weights(N_out, K_in, seed=2)
    dy = W.grads(M_tok, N_out, seed=3)
    M, N, K = PL.pass_dims(pass_, M_tok, K_in, N_out)
    A, B = PL.quantize_pass(recipe, pass_, to_gpu_bf16(x), to_gpu_bf16(w), to_gpu_bf16(dy))
    oa, ob = pass_operands(recipe, pass_, x=x, w=w, dy=dy)
    ah, bh = oa.dequant(), ob.dequant()
    cref, bnd = gemm_ref(ah, bh)
    extra = fp8_dot_unit_bound(ah, bh)
    for out_dtype in (torch.float32, torch.bfloat16):
        C = PL.gemm(recipe, pass_, A, B, M, N, K, out_dtype=out_dtype)
        _sync()
        c = out_to_np(C)
        ok, tol, err = check_gemm(c, cref, bnd, out_dtype == torch.bfloat16, extra)
        if not ok.all():
            i = tuple(np.argwhere(~ok)[0])
            pytest.fail(f"{out_dtype}: {(~ok).sum()} of {ok.size} outside bound; first {i}: got {c[i]} "
                        f"want {cref[i]} tol {tol[i]}")


@pytest.mark.parametrize("recipe", PAIRINGS)
def test_gemm_pairing_block_scales(recipe):
    """Random E4M3 codes with a different scale (2^-40 .. 2^40 times a random
    significand) on every block of A and B: within the bound only if each
    128-long slice of every output gets exactly its own two blocks' scales."""
    two = recipe.endswith("2d2d")
    M, N, K = 384, 256, 1024
    rng = np.random.default_rng(72)
    qa = rng.integers(0, 256, (M, K)).astype(np.uint8)
    qb = rng.integers(0, 256, (N, K)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0
    qb[(qb & 0x7F) == 0x7F] = 0

    def scales(rows):
        shp = (rows // 128 if two else rows, K // 128)
        return (np.ldexp(1.0, rng.integers(-40, 40, shp)) * rng.uniform(1, 2, shp)).astype(np.float32)

    sa, sb = scales(M), scales(N)
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    rec = PL.RECIPES[recipe]
    for layout in (P.PBS_FPROP, P.PBS_DGRAD, P.PBS_WGRAD):   # the layout does not change the block shapes
        P.pbs_gemm(rec, layout, M, N, K, torch.from_numpy(qa).cuda(), P.PBS_FMT_E4M3, torch.from_numpy(sa).cuda(),
                   None, torch.from_numpy(qb).cuda(), P.PBS_FMT_E4M3, torch.from_numpy(sb).cuda(), None, C,
                   P.PBS_FMT_F32)
        _sync()
        ah, bh = R.dequant_block128(qa, sa, two), R.dequant_block128(qb, sb, two)
        cref, bnd = gemm_ref(ah, bh)
        ok, tol, err = check_gemm(out_to_np(C), cref, bnd, False, fp8_dot_unit_bound(ah, bh))
        assert ok.all(), f"layout {layout}: {(~ok).sum()} of {ok.size} outside bound"


def test_pairing_rejects():
    A = torch.zeros((144, 128), dtype=torch.uint8, device="cuda")
    S = torch.ones((144,), dtype=torch.float32, device="cuda")
    C = torch.empty((144, 144), dtype=torch.float32, device="cuda")
    with pytest.raises(P.PBSError):       # 2D2D needs M, N multiples of 128
        P.pbs_gemm(P.PBS_RECIPE_FP8_BLOCK128_2D2D, P.PBS_FPROP, 144, 144, 128, A, P.PBS_FMT_E4M3, S, None, A,
                   P.PBS_FMT_E4M3, S, None, C, P.PBS_FMT_F32)
    x = torch.zeros((128, 128), dtype=torch.bfloat16, device="cuda")
    c = torch.empty((128, 128), dtype=torch.uint8, device="cuda")
    with pytest.raises(P.PBSError):       # no 2D blocks in the 1D1D pairing
        P.pbs_cast(P.PBS_RECIPE_FP8_BLOCK128_1D1D, x, 128, 128, P.PBS_FMT_E4M3, P.PBS_ROW, 1, 0, 0, None, None, c,
                   S, None, None)
