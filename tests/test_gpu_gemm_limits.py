"""GEMM operands larger than 4 GiB, against the oracle on sampled outputs.

The GEMM kernels fetch a K-major tile's rows through one buffer resource
whose range runs from the tile's first row to the operand's end, clamped to
2^32 - 1 bytes, and an MN-major stage's 64 rows through a resource based at
that stage; the lane offsets stay 32-bit.  Operands past 4 GiB exercise the
clamped range (the first tiles) and resource bases beyond the first 4 GiB
(the later tiles and stages):

* per-tensor FP8 Fprop with A of 262,400 x 16,384 E4M3 codes (4.30 GB):
  rows of the first tile, rows on either side of the 4 GiB line and of the
  last tile are checked against the oracle;
* BF16 Dgrad with B = W stored [K, N] of 131,200 x 16,384 values (4.30 GB),
  read MN-major, the last K stages beyond 4 GiB: columns of the first and
  last column tiles are checked.

Inputs are torch-seeded codes made on the device; the oracle gets the same
input bytes copied back (sampled rows or columns only) and decodes them
itself.  The bound is the parity tests' (the stated bound, the 8-bit
instruction's term for FP8, one bf16 ulp of the output).
"""
import numpy as np
import pytest
import torch

import precision_block_scaled_amd as P
from oracle.formats import E4M3, bf16_to_f32
from oracle.gemm_ref import check_gemm, fp8_dot_unit_bound, gemm_ref
from tests.gpu_util import out_to_np, scalar_gpu

pytestmark = pytest.mark.gpu

GIB4 = 1 << 32


def _fail_report(ok, c, cref, tol, where):
    i = tuple(np.argwhere(~ok)[0])
    return f"{where}: {(~ok).sum()} of {ok.size} outside bound; first {i}: got {c[i]} want {cref[i]} tol {tol[i]}"


def test_fp8_fprop_with_a_over_4gib():
    M, N, K = 262400, 256, 16384
    assert M * K > GIB4
    g = torch.Generator(device="cuda").manual_seed(11)
    # E4M3 codes of magnitude 0.5 .. 2.25 (exponent fields 6-8) with random signs
    a = torch.randint(0x30, 0x41, (M, K), dtype=torch.uint8, device="cuda", generator=g)
    a |= (torch.randint(0, 2, (M, K), dtype=torch.uint8, device="cuda", generator=g) << 7)
    b = torch.randint(0x30, 0x41, (N, K), dtype=torch.uint8, device="cuda", generator=g)
    b |= (torch.randint(0, 2, (N, K), dtype=torch.uint8, device="cuda", generator=g) << 7)
    one = scalar_gpu(np.float32(1.0))
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    P.pbs_gemm(P.PBS_RECIPE_FP8_CURRENT, P.PBS_FPROP, M, N, K, a, P.PBS_FMT_E4M3, None, one, b, P.PBS_FMT_E4M3,
               None, one, c, P.PBS_FMT_BF16)
    torch.cuda.synchronize()
    line = GIB4 // K                               # first row whose bytes start at or past 4 GiB
    rows = sorted({0, 1, 255, 256, line - 257, line - 1, line, line + 1, M - 257, M - 256, M - 1})
    idx = torch.tensor(rows, device="cuda")
    a_hat = E4M3.decode(a.index_select(0, idx).cpu().numpy())
    b_hat = E4M3.decode(b.cpu().numpy())
    del a
    cref, bnd = gemm_ref(a_hat, b_hat)
    extra = fp8_dot_unit_bound(a_hat, b_hat)
    got = out_to_np(c.index_select(0, idx))
    ok, tol, _ = check_gemm(got, cref, bnd, True, extra)
    assert ok.all(), _fail_report(ok, got, cref, tol, f"rows {rows}")


def test_bf16_dgrad_with_b_over_4gib():
    M, N, K = 256, 16384, 131200
    assert K * N * 2 > GIB4
    g = torch.Generator(device="cuda").manual_seed(12)
    dy = torch.randn((M, K), dtype=torch.float32, device="cuda", generator=g).to(torch.bfloat16)
    w = torch.empty((K, N), dtype=torch.bfloat16, device="cuda")        # W stored [K, N]: Dgrad's B
    for k0 in range(0, K, 8192):                                          # fill in slices (fp32 temporaries)
        k1 = min(K, k0 + 8192)
        w[k0:k1] = (torch.randn((k1 - k0, N), dtype=torch.float32, device="cuda", generator=g) * 0.02).to(
            torch.bfloat16)
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    P.pbs_gemm(P.PBS_RECIPE_BF16, P.PBS_DGRAD, M, N, K, dy, P.PBS_FMT_BF16, None, None, w, P.PBS_FMT_BF16, None,
               None, c, P.PBS_FMT_BF16)
    torch.cuda.synchronize()
    cols = [0, 1, 127, 255, 256, N - 257, N - 256, N - 2, N - 1]
    idx = torch.tensor(cols, device="cuda")
    a_hat = bf16_to_f32(dy.view(torch.int16).cpu().numpy().view(np.uint16))
    b_hat = bf16_to_f32(w.index_select(1, idx).contiguous().view(torch.int16).cpu().numpy().view(np.uint16)).T
    del w
    cref, bnd = gemm_ref(a_hat, b_hat)
    got = out_to_np(c.index_select(1, idx))
    ok, tol, _ = check_gemm(got, cref, bnd, True)
    assert ok.all(), _fail_report(ok, got, cref, tol, f"columns {cols}")
