"""GPU parity for sub-channel FP8 with power-of-two block scales (1x128
activation and gradient blocks, 128x128 weight blocks, MXFP8's exponent
rule per block) through the C ABI.

Casts must match the oracle bit for bit: E4M3 codes, and every 32-bit scale
word must hold the oracle's E8M0 code in each of its four bytes.  GEMMs run
on the scaled matrix instruction and must lie within the FP8 bound
(|err| <= 1e-5 * sum_k |a_k b_k| plus the 8-wide dot unit's term, + 1 bf16
ulp for bf16 outputs) of the fp64 product of the oracle-dequantized
operands.
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
from tests.gpu_util import to_gpu_bf16, to_np_u8, out_to_np, first_mismatch

pytestmark = pytest.mark.gpu

RECIPE = "fp8_block128_pow2"
CAST_CASES = [  # (src, orient, pass): every copy the three GEMMs consume
    ("x", "row", "fprop"), ("w", "row", "fprop"), ("w", "col", "dgrad"), ("dy", "row", "dgrad"),
    ("x", "col", "wgrad"), ("dy", "col", "wgrad")]


def _sync():
    torch.cuda.synchronize()


def words(codes):
    """The stored scale words for E8M0 codes: the code in all four bytes."""
    return np.asarray(codes, dtype=np.uint32) * np.uint32(0x01010101)


def gpu_words(t):
    return t.detach().cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("src,orient,pass_", CAST_CASES)
@pytest.mark.parametrize("shape", [(256, 384), (384, 128), (1152, 640)])
def test_cast_pow2(src, orient, pass_, shape):
    gen = {"x": W.activations, "w": W.weights, "dy": W.grads}[src]
    x = gen(*shape, seed=81)
    q = PL.quantize(RECIPE, to_gpu_bf16(x), src, orient, pass_)
    _sync()
    want = quantize_operand(RECIPE, src, orient, x, pass_)
    assert q.weight_2d == want.weight_2d
    assert first_mismatch(gpu_words(q.scales), words(want.scale)) is None
    assert first_mismatch(to_np_u8(q.codes), want.codes) is None


@pytest.mark.parametrize("w2d", [False, True])
def test_cast_pow2_both_copies_one_read_and_extreme_blocks(w2d):
    """orient_mask = ROW | COL (one read, both copies) on a tensor with a
    tiny block, a huge block and an all-zero block (with a -0)."""
    from oracle.formats import bf16_to_f32
    x = W.activations(256, 384, seed=82)
    t = bf16_to_f32(x).copy()
    t[:128, :128] *= np.float32(2.0 ** -110)
    t[128:, 128:256] *= np.float32(2.0 ** 100)
    t[:128, 256:] = 0.0
    t[5, 300] = -0.0
    x = W.f32_to_bf16_bits(t)
    R_, C_ = x.shape
    xg = to_gpu_bf16(x)
    rc = torch.empty((R_, C_), dtype=torch.uint8, device="cuda")
    cc = torch.empty((C_, R_), dtype=torch.uint8, device="cuda")
    rs = torch.empty(((R_ // 128) if w2d else R_, C_ // 128), dtype=torch.int32, device="cuda")
    cs = torch.empty(((C_ // 128) if w2d else C_, R_ // 128), dtype=torch.int32, device="cuda")
    P.pbs_cast(P.PBS_RECIPE_FP8_BLOCK128_POW2, xg, R_, C_, P.PBS_FMT_E4M3, P.PBS_ROW | P.PBS_COL, int(w2d), 0, 0,
               None, None, rc, rs, cc, cs)
    _sync()
    for orient, codes, sc in (("row", rc, rs), ("col", cc, cs)):
        wc, we = R.quantize_block128_pow2(x, orient, weight_2d=w2d)
        assert first_mismatch(to_np_u8(codes), wc) is None, orient
        assert first_mismatch(gpu_words(sc), words(we)) is None, orient


GEMM_DIMS = [(256, 384, 512), (272, 384, 256), (256, 256, 1536), (528, 256, 2304), (256, 384, 128),
             (400, 512, 640)]


def tensor_shapes(pass_, M, N, K):
    return {"fprop": (M, K, N), "dgrad": (M, N, K), "wgrad": (K, M, N)}[pass_]


@pytest.mark.parametrize("dims", GEMM_DIMS)
@pytest.mark.parametrize("pass_", ["fprop", "dgrad", "wgrad"])
def test_gemm_pow2_parity(dims, pass_):
    M_tok, K_in, N_out = tensor_shapes(pass_, *dims)
    x = W.activations(M_tok, K_in, seed=1)
    w = W.weights(N_out, K_in, seed=2)
    dy = W.grads(M_tok, N_out, seed=3)
    M, N, K = PL.pass_dims(pass_, M_tok, K_in, N_out)
    A, B = PL.quantize_pass(RECIPE, pass_, to_gpu_bf16(x), to_gpu_bf16(w), to_gpu_bf16(dy))
    oa, ob = pass_operands(RECIPE, pass_, x=x, w=w, dy=dy)
    ah, bh = oa.dequant(), ob.dequant()
    cref, bnd = gemm_ref(ah, bh)
    extra = fp8_dot_unit_bound(ah, bh)
    for out_dtype in (torch.float32, torch.bfloat16):
        C = PL.gemm(RECIPE, pass_, A, B, M, N, K, out_dtype=out_dtype)
        _sync()
        c = out_to_np(C)
        ok, tol, err = check_gemm(c, cref, bnd, out_dtype == torch.bfloat16, extra)
        if not ok.all():
            i = tuple(np.argwhere(~ok)[0])
            pytest.fail(f"{out_dtype}: {(~ok).sum()} of {ok.size} outside bound; first {i}: got {c[i]} "
                        f"want {cref[i]} tol {tol[i]}")


@pytest.mark.parametrize("K", [256, 1024])
def test_gemm_pow2_block_scales(K):
    """Random E4M3 codes with a different E8M0 code (127 +- 40) on every block
    of A and B: within the bound only if each 128-long slice of every output
    gets exactly its own two blocks' powers of two (B in 128x128 blocks for
    Fprop / Dgrad, 1x128 for Wgrad)."""
    M, N = 384, 256
    rng = np.random.default_rng(83)
    qa = rng.integers(0, 256, (M, K)).astype(np.uint8)
    qb = rng.integers(0, 256, (N, K)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0
    qb[(qb & 0x7F) == 0x7F] = 0
    ea = rng.integers(87, 168, (M, K // 128)).astype(np.uint8)
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    rec = PL.RECIPES[RECIPE]
    for layout in (P.PBS_FPROP, P.PBS_DGRAD, P.PBS_WGRAD):
        two = layout != P.PBS_WGRAD
        eb = rng.integers(87, 168, ((N // 128) if two else N, K // 128)).astype(np.uint8)
        sa = torch.from_numpy(words(ea).view(np.int32)).cuda()
        sb = torch.from_numpy(words(eb).view(np.int32)).cuda()
        P.pbs_gemm(rec, layout, M, N, K, torch.from_numpy(qa).cuda(), P.PBS_FMT_E4M3, sa, None,
                   torch.from_numpy(qb).cuda(), P.PBS_FMT_E4M3, sb, None, C, P.PBS_FMT_F32)
        _sync()
        ah, bh = R.dequant_block128_pow2(qa, ea, False), R.dequant_block128_pow2(qb, eb, two)
        cref, bnd = gemm_ref(ah, bh)
        ok, tol, err = check_gemm(out_to_np(C), cref, bnd, False, fp8_dot_unit_bound(ah, bh))
        assert ok.all(), f"layout {layout}: {(~ok).sum()} of {ok.size} outside bound"


def test_pow2_rejects():
    A = torch.zeros((144, 128), dtype=torch.uint8, device="cuda")
    S = torch.ones((144,), dtype=torch.int32, device="cuda")
    C = torch.empty((144, 144), dtype=torch.float32, device="cuda")
    with pytest.raises(P.PBSError):       # 128x128 weight blocks need N % 128 == 0
        P.pbs_gemm(P.PBS_RECIPE_FP8_BLOCK128_POW2, P.PBS_FPROP, 144, 144, 128, A, P.PBS_FMT_E4M3, S, None, A,
                   P.PBS_FMT_E4M3, S, None, C, P.PBS_FMT_F32)
    S8 = torch.ones((600,), dtype=torch.uint8, device="cuda")
    with pytest.raises(P.PBSError):       # scale words must be 4-byte aligned
        P.pbs_gemm(P.PBS_RECIPE_FP8_BLOCK128_POW2, P.PBS_WGRAD, 144, 144, 128, A, P.PBS_FMT_E4M3,
                   S8[1:].data_ptr(), None, A, P.PBS_FMT_E4M3, S, None, C, P.PBS_FMT_F32)
    x = torch.zeros((128, 128), dtype=torch.bfloat16, device="cuda")
    c = torch.empty((128, 128), dtype=torch.uint8, device="cuda")
    with pytest.raises(P.PBSError):       # E4M3 only
        P.pbs_cast(P.PBS_RECIPE_FP8_BLOCK128_POW2, x, 128, 128, P.PBS_FMT_E5M2, P.PBS_ROW, 0, 0, 0, None, None, c,
                   S, None, None)
