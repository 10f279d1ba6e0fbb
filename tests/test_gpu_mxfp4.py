"""GPU parity for MXFP4 (E2M1 values, E8M0 scale per 32) through the C ABI.

Casts (row, col and two-copy kernels; Hadamard transform on Wgrad
operands; stochastic rounding of dY) must match the oracle bit for bit;
GEMMs on the scaled matrix instruction with E2M1 inputs must lie within
|err| <= 1e-5 * sum_k |a_k b_k| (+ 1 bf16 ulp for bf16 outputs) of the
fp64 product of the oracle-dequantized operands.
"""
import numpy as np
import pytest
import torch

import workloads as W
import precision_block_scaled_amd as P
from precision_block_scaled_amd import pipeline as PL
from oracle import recipes as R
from oracle.formats import bf16_to_f32
from oracle.gemm_ref import gemm_ref, check_gemm
from oracle.passes import pass_operands, quantize_operand
from tests.gpu_util import to_gpu_bf16, to_np_u8, out_to_np, first_mismatch

pytestmark = pytest.mark.gpu


def _sync():
    torch.cuda.synchronize()


CAST_CASES = [  # (src, orient, pass): every copy the three GEMMs consume
    ("x", "row", "fprop"), ("w", "row", "fprop"), ("w", "col", "dgrad"), ("dy", "row", "dgrad"),
    ("x", "col", "wgrad"), ("dy", "col", "wgrad")]


@pytest.mark.parametrize("src,orient,pass_", CAST_CASES)
@pytest.mark.parametrize("shape", [(256, 512), (160, 96), (32, 32)])
def test_cast_mxfp4(src, orient, pass_, shape):
    gen = {"x": W.activations, "w": W.weights, "dy": W.grads}[src]
    x = gen(*shape, seed=41)
    q = PL.quantize("mxfp4", to_gpu_bf16(x), src, orient, pass_)
    _sync()
    want = quantize_operand("mxfp4", src, orient, x, pass_)
    assert q.tensor_scale_inv is None and want.tensor_scale_inv is None
    assert first_mismatch(to_np_u8(q.scales), want.scale) is None
    assert first_mismatch(to_np_u8(q.codes), want.codes) is None


def _cast(x, rows, cols, mask, flags=0, seed=42):
    rc = torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda") if mask & P.PBS_ROW else None
    rs = torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda") if mask & P.PBS_ROW else None
    cc = torch.empty((cols, rows // 2), dtype=torch.uint8, device="cuda") if mask & P.PBS_COL else None
    cs = torch.empty((cols, rows // 32), dtype=torch.uint8, device="cuda") if mask & P.PBS_COL else None
    P.pbs_cast(P.PBS_RECIPE_MXFP4, to_gpu_bf16(x), rows, cols, P.PBS_FMT_E2M1, mask, 0, flags, seed, None,
               None, rc, rs, cc, cs)
    _sync()
    return rc, rs, cc, cs


def _want(x, orient, sr=False, rht=False):
    t = bf16_to_f32(x)
    if rht:
        t = R.rht16_along_rows(t, 42)
    t_o = t if orient == "row" else np.ascontiguousarray(t.T)
    r = R.sr_random_for(x.shape, orient, 42) if sr else None
    return R.quantize_mxfp4(t_o, sr_random=r)


@pytest.mark.parametrize("mask", [P.PBS_ROW, P.PBS_COL, P.PBS_ROW | P.PBS_COL])
@pytest.mark.parametrize("sr", [False, True])
def test_cast_mxfp4_all_bf16_patterns(mask, sr):
    """Every finite bf16 value, through the row, col and two-copy kernels."""
    x = W.all_bf16_patterns()
    rc, rs, cc, cs = _cast(x, 256, 256, mask, P.PBS_FLAG_SR if sr else 0)
    for orient, c, s in (("row", rc, rs), ("col", cc, cs)):
        if c is None:
            continue
        codes, e8 = _want(x, orient, sr)
        assert first_mismatch(to_np_u8(s), e8) is None, orient
        assert first_mismatch(to_np_u8(c), codes) is None, orient


@pytest.mark.parametrize("sr", [False, True])
def test_cast_mxfp4_rht_col(sr):
    x = W.grads(512, 96, seed=43)
    _, _, cc, cs = _cast(x, 512, 96, P.PBS_COL, P.PBS_FLAG_RHT16 | (P.PBS_FLAG_SR if sr else 0))
    codes, e8 = _want(x, "col", sr, rht=True)
    assert first_mismatch(to_np_u8(cs), e8) is None
    assert first_mismatch(to_np_u8(cc), codes) is None


def test_cast_mxfp4_exponent_edges():
    """Block maxima at 6 * 2^k and one bf16 step above, zero and subnormal blocks, -0."""
    rows, cols = 32, 256
    t = np.zeros((rows, cols), np.float32)
    rng = np.random.default_rng(44)
    for r in range(rows):
        for b in range(cols // 32):
            k = int(rng.integers(-140, 120))
            blk = rng.uniform(-1, 1, 32).astype(np.float32) * np.float32(2.0 ** k)
            if b % 4 == 0:
                blk[3] = np.float32(6 * 2.0 ** min(k, 125))
            elif b % 4 == 1:
                blk[7] = np.float32(6 * 2.0 ** min(k, 125)) * np.float32(1 + 2 ** -7)
            elif b % 4 == 2:
                blk[:] = 0.0
                blk[5] = -0.0
            t[r, 32 * b:32 * b + 32] = blk
    x = W.f32_to_bf16_bits(t)
    rc, rs, cc, cs = _cast(x, rows, cols, P.PBS_ROW | P.PBS_COL)
    for orient, c, s in (("row", rc, rs), ("col", cc, cs)):
        codes, e8 = _want(x, orient)
        assert first_mismatch(to_np_u8(s), e8) is None, orient
        assert first_mismatch(to_np_u8(c), codes) is None, orient
    rc1, rs1, _, _ = _cast(x, rows, cols, P.PBS_ROW)
    assert (rc1 == rc).all() and (rs1 == rs).all()


def test_cast_mxfp4_rejects():
    x = torch.zeros((64, 48), dtype=torch.bfloat16, device="cuda")
    c = torch.empty((64, 24), dtype=torch.uint8, device="cuda")
    s = torch.empty((64, 2), dtype=torch.uint8, device="cuda")
    with pytest.raises(P.PBSError):       # cols not a multiple of 32
        P.pbs_cast(P.PBS_RECIPE_MXFP4, x, 64, 48, P.PBS_FMT_E2M1, P.PBS_ROW, 0, 0, 42, None, None, c, s,
                   None, None)
    with pytest.raises(P.PBSError):       # no 2D blocks for MXFP4
        P.pbs_cast(P.PBS_RECIPE_MXFP4, x, 64, 32, P.PBS_FMT_E2M1, P.PBS_ROW, 1, 0, 42, None, None, c, s,
                   None, None)
    with pytest.raises(P.PBSError):       # E2M1 only
        P.pbs_cast(P.PBS_RECIPE_MXFP4, x, 64, 32, P.PBS_FMT_E4M3, P.PBS_ROW, 0, 0, 42, None, None, c, s,
                   None, None)


# ---------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------
GEMM_DIMS = [  # (M, N, K): K = 256 (one stage), 512 (two), 1536 and 2304 (the pipelined loop),
    (256, 384, 512),  # ragged M / N
    (272, 400, 256),
    (256, 256, 1536),
    (528, 272, 2304),
]


def tensor_shapes(pass_, M, N, K):
    return {"fprop": (M, K, N), "dgrad": (M, N, K), "wgrad": (K, M, N)}[pass_]


def _run(pass_, x, w, dy, out_dtype):
    M, N, K = PL.pass_dims(pass_, x.shape[0], x.shape[1], w.shape[0])
    A, B = PL.quantize_pass("mxfp4", pass_, to_gpu_bf16(x), to_gpu_bf16(w), to_gpu_bf16(dy))
    C = PL.gemm("mxfp4", pass_, A, B, M, N, K, out_dtype=out_dtype)
    _sync()
    oa, ob = pass_operands("mxfp4", pass_, x=x, w=w, dy=dy)
    cref, bnd = gemm_ref(oa.dequant(), ob.dequant())
    return out_to_np(C), cref, bnd


@pytest.mark.parametrize("pass_", ["fprop", "dgrad", "wgrad"])
@pytest.mark.parametrize("dims", GEMM_DIMS)
def test_gemm_mxfp4_parity(pass_, dims):
    M_tok, K_in, N_out = tensor_shapes(pass_, *dims)
    x = W.activations(M_tok, K_in, seed=1)
    w = W.weights(N_out, K_in, seed=2)
    dy = W.grads(M_tok, N_out, seed=3)
    for out_dtype in (torch.float32, torch.bfloat16):
        c, cref, bnd = _run(pass_, x, w, dy, out_dtype)
        ok, tol, err = check_gemm(c, cref, bnd, out_dtype == torch.bfloat16)
        if not ok.all():
            i = tuple(np.argwhere(~ok)[0])
            pytest.fail(f"{out_dtype}: {(~ok).sum()} of {ok.size} outside bound; first {i}: got {c[i]} "
                        f"want {cref[i]} tol {tol[i]}")


def test_gemm_mxfp4_block_scales():
    """Random E2M1 codes with a different E8M0 scale (2^-40 .. 2^39) on every
    32-block of A and B: the product is within the bound only if each lane's
    scale reaches exactly its own 32 products."""
    M, N, K = 64, 96, 1024
    rng = np.random.default_rng(45)
    qa = rng.integers(0, 16, (M, K)).astype(np.uint8)
    qb = rng.integers(0, 16, (N, K)).astype(np.uint8)
    ea = rng.integers(127 - 40, 127 + 40, (M, K // 32)).astype(np.uint8)
    eb = rng.integers(127 - 40, 127 + 40, (N, K // 32)).astype(np.uint8)
    A = torch.from_numpy(R.pack_e2m1(qa)).cuda()
    B = torch.from_numpy(R.pack_e2m1(qb)).cuda()
    SA = torch.from_numpy(ea).cuda()
    SB = torch.from_numpy(eb).cuda()
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    P.pbs_gemm(P.PBS_RECIPE_MXFP4, P.PBS_FPROP, M, N, K, A, P.PBS_FMT_E2M1, SA, None, B, P.PBS_FMT_E2M1,
               SB, None, C, P.PBS_FMT_F32)
    _sync()
    ah = R.dequant_mxfp4(R.pack_e2m1(qa), ea)
    bh = R.dequant_mxfp4(R.pack_e2m1(qb), eb)
    cref, bnd = gemm_ref(ah, bh)
    ok, tol, err = check_gemm(out_to_np(C), cref, bnd, False)
    assert ok.all(), f"{(~ok).sum()} of {ok.size} outside bound"


def test_gemm_mxfp4_deterministic_and_rejects():
    x = W.activations(256, 512, seed=1)
    w = W.weights(384, 512, seed=2)
    dy = W.grads(256, 384, seed=3)
    c1 = _run("wgrad", x, w, dy, torch.float32)[0]
    c2 = _run("wgrad", x, w, dy, torch.float32)[0]
    assert (c1 == c2).all()
    A = torch.zeros((32, 64), dtype=torch.uint8, device="cuda")
    S = torch.zeros((32, 4), dtype=torch.uint8, device="cuda")
    C = torch.empty((32, 32), dtype=torch.float32, device="cuda")
    with pytest.raises(P.PBSError):       # K = 128 is not a multiple of 256
        P.pbs_gemm(P.PBS_RECIPE_MXFP4, P.PBS_FPROP, 32, 32, 128, A, P.PBS_FMT_E2M1, S, None, A,
                   P.PBS_FMT_E2M1, S, None, C, P.PBS_FMT_F32)
    with pytest.raises(P.PBSError):       # block scales required
        P.pbs_gemm(P.PBS_RECIPE_MXFP4, P.PBS_FPROP, 32, 32, 256, A, P.PBS_FMT_E2M1, None, None, A,
                   P.PBS_FMT_E2M1, S, None, C, P.PBS_FMT_F32)
