"""GPU parity for channel-wise FP8 (one fp32 scale per row of each copy)
through the C ABI.

Casts (row kernel in each of its register-resident sizes and the two-read
form for very long rows; column maxima + col cast + finalize) must match the
oracle bit for bit, codes and scales; GEMMs must lie within the FP8 bound
(the stated |err| <= 1e-5 * sum_k |a_k b_k| plus the 8-wide dot unit's term,
+ 1 bf16 ulp for bf16 outputs) of the fp64 product of the oracle-dequantized
operands.
"""
import numpy as np
import pytest
import torch

import workloads as W
import precision_block_scaled_amd as P
from precision_block_scaled_amd import pipeline as PL
from oracle import recipes as R
from oracle.formats import bf16_to_f32
from oracle.gemm_ref import gemm_ref, check_gemm, fp8_dot_unit_bound
from oracle.passes import pass_operands, quantize_operand
from tests.gpu_util import to_gpu_bf16, to_np_u8, to_np_f32, out_to_np, first_mismatch

pytestmark = pytest.mark.gpu

REC = P.PBS_RECIPE_FP8_CHANNEL


def _sync():
    torch.cuda.synchronize()


def _cast(x, rows, cols, mask):
    dev = "cuda"
    rc = torch.empty((rows, cols), dtype=torch.uint8, device=dev) if mask & P.PBS_ROW else None
    rs = torch.full((rows,), -7.0, dtype=torch.float32, device=dev) if mask & P.PBS_ROW else None
    cc = torch.empty((cols, rows), dtype=torch.uint8, device=dev) if mask & P.PBS_COL else None
    cs = torch.full((cols,), -7.0, dtype=torch.float32, device=dev) if mask & P.PBS_COL else None
    xg = to_gpu_bf16(x)
    P.pbs_cast(REC, xg, rows, cols, P.PBS_FMT_E4M3, mask, 0, 0, 0, None, None, rc, rs, cc, cs)
    _sync()
    return rc, rs, cc, cs


def _check(x, orient, codes, scales):
    want_c, want_s = R.quantize_channel(x, orient)
    assert first_mismatch(to_np_f32(scales).view(np.uint32), want_s.view(np.uint32)) is None, orient
    assert first_mismatch(to_np_u8(codes), want_c) is None, orient


CAST_CASES = [  # (src, orient, pass): every copy the three GEMMs consume
    ("x", "row", "fprop"), ("w", "row", "fprop"), ("w", "col", "dgrad"), ("dy", "row", "dgrad"),
    ("x", "col", "wgrad"), ("dy", "col", "wgrad")]


@pytest.mark.parametrize("src,orient,pass_", CAST_CASES)
@pytest.mark.parametrize("shape", [(256, 512), (160, 96), (272, 1040), (16, 16)])
def test_cast_channel(src, orient, pass_, shape):
    gen = {"x": W.activations, "w": W.weights, "dy": W.grads}[src]
    x = gen(*shape, seed=51)
    q = PL.quantize("fp8_channel", to_gpu_bf16(x), src, orient, pass_)
    _sync()
    want = quantize_operand("fp8_channel", src, orient, x, pass_)
    assert first_mismatch(to_np_f32(q.scales).view(np.uint32), want.scale.view(np.uint32)) is None
    assert first_mismatch(to_np_u8(q.codes), want.codes) is None


# one row length per row-kernel variant (wave teams of 1-8 segments per lane,
# workgroup teams of 4-16, the two-read form), ragged lengths included
@pytest.mark.parametrize("cols", [16, 1024, 1040, 2048, 4096, 8192, 8208, 16384, 32768, 65536, 65552])
def test_cast_channel_row_lengths(cols):
    x = W.grads(16, cols, seed=52)
    rc, rs, _, _ = _cast(x, 16, cols, P.PBS_ROW)
    _check(x, "row", rc, rs)


@pytest.mark.parametrize("rows,cols", [(16, 16), (48, 512), (272, 1040), (4112, 48), (1040, 528)])
def test_cast_channel_col_shapes(rows, cols):
    """Column maxima over ragged row chunks and partial 512-column groups."""
    x = W.activations(rows, cols, seed=53)
    _, _, cc, cs = _cast(x, rows, cols, P.PBS_COL)
    _check(x, "col", cc, cs)


def test_cast_channel_both_and_all_bf16_patterns():
    x = W.all_bf16_patterns()
    rc, rs, cc, cs = _cast(x, 256, 256, P.PBS_ROW | P.PBS_COL)
    _check(x, "row", rc, rs)
    _check(x, "col", cc, cs)
    rc1, rs1, _, _ = _cast(x, 256, 256, P.PBS_ROW)
    _, _, cc1, cs1 = _cast(x, 256, 256, P.PBS_COL)
    assert (rc1 == rc).all() and (rs1 == rs).all() and (cc1 == cc).all() and (cs1 == cs).all()


def test_cast_channel_zero_rows_outliers_and_overflow():
    """All-zero rows and columns (scale 1), a +-0 mix, one outlier per row,
    and amax small enough that 448 / amax overflows (scale FLT_MAX)."""
    rows, cols = 64, 256
    t = bf16_to_f32(W.activations(rows, cols, seed=54)).copy()
    t[3, :] = 0.0
    t[3, 5] = -0.0
    t[10, 200] = 3.0e38
    t[11, :] = np.float32(2.0 ** -130)       # subnormal row: 448 / amax overflows
    t[12, 9] = -1.0e-40
    t[:, 7] = 0.0
    x = W.f32_to_bf16_bits(t)
    rc, rs, cc, cs = _cast(x, rows, cols, P.PBS_ROW | P.PBS_COL)
    _check(x, "row", rc, rs)
    _check(x, "col", cc, cs)
    s = to_np_f32(rs)
    assert s[3] == 1.0 and to_np_f32(cs)[7] == 1.0
    assert s[11] == np.float32(1.0) / np.finfo(np.float32).max


def test_cast_channel_empty():
    """Rows of length 0 and columns of length 0 get scale 1 (the zero-amax rule)."""
    x = torch.empty((0,), dtype=torch.bfloat16, device="cuda")
    dummy = torch.empty((16,), dtype=torch.uint8, device="cuda")
    rs = torch.full((32,), -7.0, dtype=torch.float32, device="cuda")
    P.pbs_cast(REC, x, 32, 0, P.PBS_FMT_E4M3, P.PBS_ROW, 0, 0, 0, None, None, dummy, rs, None, None)
    cs = torch.full((48,), -7.0, dtype=torch.float32, device="cuda")
    P.pbs_cast(REC, x, 0, 48, P.PBS_FMT_E4M3, P.PBS_COL, 0, 0, 0, None, None, None, None, dummy, cs)
    _sync()
    assert (to_np_f32(rs) == 1.0).all() and (to_np_f32(cs) == 1.0).all()
    want = R.quantize_channel(np.zeros((32, 0), np.uint16), "row")[1]
    assert (want == 1.0).all()


def test_cast_channel_rejects():
    x = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    c = torch.empty((64, 64), dtype=torch.uint8, device="cuda")
    s = torch.empty((65,), dtype=torch.float32, device="cuda")
    with pytest.raises(P.PBSError):       # E4M3 only
        P.pbs_cast(REC, x, 64, 64, P.PBS_FMT_E5M2, P.PBS_ROW, 0, 0, 0, None, None, c, s, None, None)
    with pytest.raises(P.PBSError):       # scales required
        P.pbs_cast(REC, x, 64, 64, P.PBS_FMT_E4M3, P.PBS_ROW, 0, 0, 0, None, None, c, None, None, None)
    with pytest.raises(P.PBSError):       # no 2D blocks
        P.pbs_cast(REC, x, 64, 64, P.PBS_FMT_E4M3, P.PBS_ROW, 1, 0, 0, None, None, c, s, None, None)
    with pytest.raises(P.PBSError):       # no fused per-tensor amax
        P.pbs_cast(REC, x, 64, 64, P.PBS_FMT_E4M3, P.PBS_ROW, 0, 0, 0, None, s[:1], c, s, None, None)


# ---------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------
GEMM_DIMS = [  # (M, N, K): one stage, the pipelined loop, ragged M and N
    (256, 384, 512),
    (272, 400, 128),
    (256, 256, 1536),
    (528, 272, 2304),
]


def tensor_shapes(pass_, M, N, K):
    return {"fprop": (M, K, N), "dgrad": (M, N, K), "wgrad": (K, M, N)}[pass_]


def _run(pass_, x, w, dy, out_dtype):
    M, N, K = PL.pass_dims(pass_, x.shape[0], x.shape[1], w.shape[0])
    A, B = PL.quantize_pass("fp8_channel", pass_, to_gpu_bf16(x), to_gpu_bf16(w), to_gpu_bf16(dy))
    C = PL.gemm("fp8_channel", pass_, A, B, M, N, K, out_dtype=out_dtype)
    _sync()
    oa, ob = pass_operands("fp8_channel", pass_, x=x, w=w, dy=dy)
    ah, bh = oa.dequant(), ob.dequant()
    cref, bnd = gemm_ref(ah, bh)
    return out_to_np(C), cref, bnd, fp8_dot_unit_bound(ah, bh)


@pytest.mark.parametrize("pass_", ["fprop", "dgrad", "wgrad"])
@pytest.mark.parametrize("dims", GEMM_DIMS)
def test_gemm_channel_parity(pass_, dims):
    M_tok, K_in, N_out = tensor_shapes(pass_, *dims)
    x = W.activations(M_tok, K_in, seed=1)
    w = W.weights(N_out, K_in, seed=2)
    dy = W.grads(M_tok, N_out, seed=3)
    for out_dtype in (torch.float32, torch.bfloat16):
        c, cref, bnd, extra = _run(pass_, x, w, dy, out_dtype)
        ok, tol, err = check_gemm(c, cref, bnd, out_dtype == torch.bfloat16, extra)
        if not ok.all():
            i = tuple(np.argwhere(~ok)[0])
            pytest.fail(f"{out_dtype}: {(~ok).sum()} of {ok.size} outside bound; first {i}: got {c[i]} "
                        f"want {cref[i]} tol {tol[i]}")


def test_gemm_channel_row_scales():
    """Random E4M3 codes with a different scale (2^-40 .. 2^40) on every row
    of A and of B: within the bound only if output (m, n) gets exactly
    a_scale[m] * b_scale[n]."""
    M, N, K = 304, 272, 512
    rng = np.random.default_rng(55)
    qa = rng.integers(0, 256, (M, K)).astype(np.uint8)
    qb = rng.integers(0, 256, (N, K)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0           # no NaN codes
    qb[(qb & 0x7F) == 0x7F] = 0
    sa = np.ldexp(1.0, rng.integers(-40, 40, M)).astype(np.float32) * rng.uniform(1, 2, M).astype(np.float32)
    sb = np.ldexp(1.0, rng.integers(-40, 40, N)).astype(np.float32) * rng.uniform(1, 2, N).astype(np.float32)
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    P.pbs_gemm(REC, P.PBS_FPROP, M, N, K, torch.from_numpy(qa).cuda(), P.PBS_FMT_E4M3, torch.from_numpy(sa).cuda(),
               None, torch.from_numpy(qb).cuda(), P.PBS_FMT_E4M3, torch.from_numpy(sb).cuda(), None, C,
               P.PBS_FMT_F32)
    _sync()
    ah, bh = R.dequant_channel(qa, sa), R.dequant_channel(qb, sb)
    cref, bnd = gemm_ref(ah, bh)
    ok, tol, err = check_gemm(out_to_np(C), cref, bnd, False, fp8_dot_unit_bound(ah, bh))
    assert ok.all(), f"{(~ok).sum()} of {ok.size} outside bound"


def test_gemm_channel_rejects():
    A = torch.zeros((32, 128), dtype=torch.uint8, device="cuda")
    S = torch.ones((40,), dtype=torch.float32, device="cuda")
    C = torch.empty((32, 32), dtype=torch.float32, device="cuda")
    with pytest.raises(P.PBSError):       # scales not 16-byte aligned
        P.pbs_gemm(REC, P.PBS_FPROP, 32, 32, 128, A, P.PBS_FMT_E4M3, S[1:], None, A, P.PBS_FMT_E4M3, S, None,
                   C, P.PBS_FMT_F32)
    with pytest.raises(P.PBSError):       # scales required
        P.pbs_gemm(REC, P.PBS_FPROP, 32, 32, 128, A, P.PBS_FMT_E4M3, None, None, A, P.PBS_FMT_E4M3, S, None,
                   C, P.PBS_FMT_F32)
    with pytest.raises(P.PBSError):       # E4M3 only
        P.pbs_gemm(REC, P.PBS_FPROP, 32, 32, 128, A, P.PBS_FMT_E5M2, S, None, A, P.PBS_FMT_E4M3, S, None,
                   C, P.PBS_FMT_F32)
