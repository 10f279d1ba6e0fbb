"""The measured description of the 8-bit matrix instruction (tests/
fp8_dot_unit.py) against a second, scalar statement of it in exact
rationals, and against the oracle's tolerance for FP8-instruction GEMMs.

The oracle accepts an FP8-instruction GEMM output when |C - C_ref| <=
1e-5 * sum|a b| + 2**-10 * sum over aligned 8-groups of max|a b| (plus a bf16
ulp for bf16 output).  These CPU tests show, from the description alone,
that (1) the second term is needed: the instruction's truncation alone
exceeds the first term on outlier-heavy inputs, and (2) it suffices on the
inputs the tests and the benchmark use.  The GPU tests
(test_gpu_fp8_dot_unit.py) check the instruction against the description bit
for bit.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import workloads as W
from oracle.formats import E4M3, E5M2
from oracle.gemm_ref import REL_TOL, fp8_dot_unit_bound, gemm_ref
from tests.fp8_dot_unit import dot_unit_gemm, group_sums

FMT = {"e4m3": E4M3, "e5m2": E5M2}


def _frac_to_f32(x):
    """Round a Fraction to the nearest float32 (ties to even), by exact search."""
    if x == 0:
        return Fraction(0)
    sgn = -1 if x < 0 else 1
    a = abs(x)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 23)
    q, r = divmod(a, ulp)
    if r * 2 > ulp or (r * 2 == ulp and q % 2 == 1):
        q += 1
    return sgn * q * ulp


def _scalar_model(a, b, fa, fb):
    """The description, one output at a time, in exact rationals."""
    emin = {"e4m3": -6, "e5m2": -14}
    ex = lambda v, f: max(math.frexp(float(abs(v)))[1] - 1, emin[f])
    acc = Fraction(0)
    K = len(a)
    for s0 in range(0, K, 16):
        step = Fraction(0)
        for g0 in (s0, s0 + 8):
            ps = [(Fraction(float(a[k])), Fraction(float(b[k]))) for k in range(g0, g0 + 8)
                  if a[k] != 0 and b[k] != 0]
            if not ps:
                continue
            emax = max(ex(x, fa) + ex(y, fb) for x, y in ps)
            q = Fraction(2) ** (emax - 13)
            for x, y in ps:
                t = (x * y) / q
                step += (math.floor(t) if t >= 0 else -math.floor(-t)) * q
        acc = _frac_to_f32(acc + step)
    return float(acc)


def _codes(rng, fmt, shape, outliers=0.0):
    F = FMT[fmt]
    v = rng.standard_normal(shape) * 2.0
    if outliers:
        v = np.where(rng.random(shape) < outliers, v * 100.0, v)
    v = np.clip(v, -F.max_value, F.max_value)
    return F.decode(F.encode(v))


@pytest.mark.parametrize("fa,fb,seed", [("e4m3", "e4m3", 0), ("e5m2", "e4m3", 1), ("e4m3", "e5m2", 2)])
def test_vectorized_description_equals_scalar_restatement(fa, fb, seed):
    rng = np.random.default_rng(seed)
    a = _codes(rng, fa, (4, 64), outliers=0.05)
    b = _codes(rng, fb, (3, 64), outliers=0.05)
    a[0, :5] = 0.0                                # zero products and -0
    b[1, 7] = -0.0
    a[2, 9] = 2.0 ** -9 if fa == "e4m3" else 2.0 ** -16     # subnormal operands
    a[3, 17:19] = FMT[fa].decode(np.array([1, 3]))               # a group led by subnormals
    a[3, 16] = a[3, 20:24] = 0.0
    got = dot_unit_gemm(a, b, fa, fb)
    for i in range(4):
        for j in range(3):
            assert got[i, j] == np.float32(_scalar_model(a[i], b[j], fa, fb)), (i, j)


def _one(prods, K=128, fa="e4m3", fb="e4m3"):
    a = np.zeros((1, K))
    b = np.zeros((1, K))
    for k, x, y in prods:
        a[0, k], b[0, k] = x, y
    return float(dot_unit_gemm(a, b, fa, fb)[0, 0])


def test_description_consequences_by_hand():
    """Values that follow from the description by hand.  448 * 448 = 200704
    has exponent sum 8 + 8 = 16, so its group keeps multiples of 2**3."""
    big = (0, 448.0, 448.0)
    assert _one([big, (1, 4.0, 2.0)]) == 200712.0          # 8 = 2**3: kept
    assert _one([big, (1, 1.0, 4.0)]) == 200704.0          # 4 < 2**3: lost
    assert _one([big, (1, 3.0, 4.0)]) == 200712.0          # 12 -> 8
    assert _one([big, (1, -3.0, 4.0)]) == 200696.0         # -12 -> -8 (toward zero)
    assert _one([big, (1, -1.0, 4.0)]) == 200704.0         # -4 -> 0
    assert _one([(7, 448.0, 448.0), (6, 1.0, 4.0)]) == 200704.0   # same aligned group
    assert _one([(7, 448.0, 448.0), (8, 1.0, 4.0)]) == 200708.0   # next group: kept
    assert _one([(8, 448.0, 448.0), (15, 1.0, 4.0)]) == 200704.0
    assert _one([(8, 448.0, 448.0), (16, 1.0, 4.0)]) == 200708.0
    # 240 * 240 = 57600, exponent sum 14: multiples of 2 survive (3 -> 2)
    assert _one([(0, 240.0, 240.0), (1, 1.0, 2.0), (2, 1.0, 3.0)]) == 57604.0
    # a zero operand does not set the group's exponent
    assert _one([(0, 448.0, 0.0), (1, 1.0, 4.0)]) == 4.0
    # a subnormal operand counts with the smallest normal exponent: 2**-9 (an
    # E4M3 subnormal) x 448 has exponent sum -6 + 8 = 2, so the group keeps
    # multiples of 2**-11: 2**-6 x 2**-6 = 2**-12 is lost, 2**-6 x 2**-5 kept
    assert _one([(0, 2.0 ** -9, 448.0), (1, 2.0 ** -6, 2.0 ** -6)]) == 0.875
    assert _one([(0, 2.0 ** -9, 448.0), (1, 2.0 ** -6, 2.0 ** -5)]) == 0.875 + 2.0 ** -11
    # E5M2 x E4M3: 57344 * 448 = 25690112 (exponent sum 23, fp32 spacing 2).
    # Two groups of one 16-index step are summed before one rounding
    # (max + 1 + 1 in one step: max + 2), a single 1 in a step is lost
    # against max (tie to even), and the step of 16 is the rounding unit.
    m = (57344.0, 448.0)
    _e5 = lambda prods: _one(prods, fa="e5m2")
    assert _e5([(0, *m), (8, 1.0, 1.0), (16, 1.0, 1.0), (24, 1.0, 1.0)]) == 25690114.0
    assert _e5([(0, *m), (8, 1.0, 1.0), (24, 1.0, 1.0)]) == 25690112.0
    assert _e5([(0, 1.0, 1.0), (8, 1.0, 1.0), (16, 1.0, 1.0), (24, *m)]) == 25690116.0
    assert _e5([(8 * g, 1.0, 1.0) for g in range(7)] + [(56, *m)]) == 25690120.0
    assert _e5([(0, *m)] + [(8 * g, 1.0, 1.0) for g in range(1, 8)]) == 25690118.0


def test_group_loss_bounded_by_oracle_term():
    """Per group the truncation loses less than 7 * 2**(e_max - 13) <= 7 *
    2**-13 * max|ab| < 2**-10 * max|ab|: checked on every group of random
    outlier-heavy operands, in exact arithmetic."""
    rng = np.random.default_rng(5)
    a = _codes(rng, "e4m3", (16, 256), outliers=0.03)
    b = _codes(rng, "e5m2", (16, 256), outliers=0.03)
    gs = group_sums(a, b, "e4m3", "e5m2")
    exact = (a[:, None, :] * b[None, :, :]).reshape(16, 16, 32, 8).sum(axis=3)   # exact: <= 8 terms, 8-bit
    mx = np.abs(a[:, None, :] * b[None, :, :]).reshape(16, 16, 32, 8).max(axis=3)
    loss = np.abs(gs - exact)
    assert (loss < 7 * 2.0 ** -13 * mx + (mx == 0)).all()
    assert (loss <= 2.0 ** -10 * mx).all()


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e4m3", "e5m2")])
def test_stated_bound_alone_fails_and_oracle_term_covers(fa, fb):
    """Adversarial groups: one large product and seven products just below
    its group's truncation step, each lost entirely (448 x 448 keeps
    multiples of 8, against products of 7; 57344 x 448 keeps multiples of
    1024, against products of 7 x 128 = 896).  The loss exceeds 1e-5 *
    sum|ab| while staying inside the 2**-10 * max term."""
    K = 512
    a = np.zeros((1, K))
    b = np.zeros((1, K))
    big_a, small_b = (448.0, 1.0) if fa == "e4m3" else (57344.0, 128.0)
    for g in range(0, K, 8):
        a[0, g], b[0, g] = big_a, 448.0
        a[0, g + 1:g + 8], b[0, g + 1:g + 8] = 7.0, small_b
    got = dot_unit_gemm(a, b, fa, fb).astype(np.float64)
    cref, base = gemm_ref(a, b)
    err = np.abs(got - cref)
    assert (err > REL_TOL * base).all()
    assert (err <= REL_TOL * base + fp8_dot_unit_bound(a, b)).all()


@pytest.mark.parametrize("recipe_fmt", [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e4m3", "e5m2")])
def test_oracle_tolerance_covers_benchmark_like_inputs(recipe_fmt):
    """On the workload's distributions (activations with outlier channels x
    100, weights N(0, 0.02^2), Student-t gradients), per-tensor-scaled FP8
    codes: the description's result lies within the oracle's tolerance,
    and on these inputs it exceeds the stated 1e-5 term somewhere."""
    from oracle import recipes as R
    fa, fb = recipe_fmt
    K = 1024
    x = W.activations(32, K, seed=41)
    w = W.weights(32, K, seed=42)
    dy = W.grads(32, K, seed=43)
    srcs = {("e4m3", "e4m3"): (x, w), ("e5m2", "e4m3"): (dy, w), ("e4m3", "e5m2"): (x, dy)}[recipe_fmt]
    ca, _, _ = R.quantize_current(srcs[0], fa, "row")
    cb, _, _ = R.quantize_current(srcs[1], fb, "row")
    a, b = FMT[fa].decode(ca), FMT[fb].decode(cb)
    got = dot_unit_gemm(a, b, fa, fb).astype(np.float64)
    cref, base = gemm_ref(a, b)
    err = np.abs(got - cref)
    assert (err <= REL_TOL * base + fp8_dot_unit_bound(a, b)).all()
    if fa == "e4m3" and fb == "e4m3":
        assert (err > REL_TOL * base).any()
