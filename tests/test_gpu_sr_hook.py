"""The device's stochastic E2M1 rounding at its exact threshold.

Stochastic rounding of gradients ("How to optimize Transformer-based models
for low-precision training", "Interpreting results for a real model") rounds
|v| up to the next E2M1 magnitude hi with probability P = (|v| - lo) /
(hi - lo).  With a 32-bit random word r the rule is: hi iff r < P * 2**32.
For integer r that is r < T with T = ceil(P * 2**32), so r = T - 1 must give
hi and r = T must give lo.  A cast meets such an r with probability about
2**-32 per element, so the test-only entry point pbs_debug_sr_encode runs
the device rounding on chosen (v, r) pairs.  T is computed here in exact
rationals from the definition; the oracle's sr_e2m1 is checked on the same
pairs.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import precision_block_scaled_amd as P
from oracle import recipes as R
from oracle.formats import E2M1

pytestmark = pytest.mark.gpu

MAGS = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def expected(v, r):
    """(code) from the definition: sign kept, |v| >= 6 -> 6, else lo / hi by r < ceil(P * 2**32)."""
    a = abs(Fraction(float(v)))
    sign = 8 if math.copysign(1.0, float(v)) < 0 else 0
    if a >= 6:
        return 7 | sign
    lo = max(i for i in range(8) if MAGS[i] <= a)
    P_ = (a - MAGS[lo]) / (MAGS[lo + 1] - MAGS[lo])
    T = math.ceil(P_ * 2 ** 32)
    return (lo + 1 if r < T else lo) | sign


def threshold(v):
    a = abs(Fraction(float(v)))
    lo = max(i for i in range(8) if MAGS[i] <= a)
    return math.ceil((a - MAGS[lo]) / (MAGS[lo + 1] - MAGS[lo]) * 2 ** 32)


def _values():
    rng = np.random.default_rng(11)
    v = [rng.uniform(0, 6, 2000), rng.uniform(0, 0.5, 500), rng.uniform(5.9, 6.0, 100),
         np.ldexp(rng.uniform(1, 2, 300), rng.integers(-40, -2, 300))]       # tiny: fractional P * 2**32
    v = np.concatenate(v).astype(np.float32)
    # values just around every grid point, and the grid points themselves
    grid = np.array([0.5, 1, 1.5, 2, 3, 4], np.float32)
    near = np.concatenate([grid, np.nextafter(grid, np.float32(0)), np.nextafter(grid, np.float32(9))])
    v = np.concatenate([v, near, np.float32([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 2.0 ** -149])])
    v = np.concatenate([v, -v])
    return v.astype(np.float32)


def _device_sr(v, r):
    n = len(v)
    vg = torch.from_numpy(np.ascontiguousarray(v, np.float32)).cuda()
    rg = torch.from_numpy(np.ascontiguousarray(r, np.uint32).view(np.int32)).cuda()
    out = torch.empty(n, dtype=torch.uint8, device="cuda")
    P.pbs_debug_sr_encode(vg, rg, out, n)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_threshold_edges():
    v = _values()
    T = np.array([threshold(x) for x in v], dtype=np.int64)
    assert (T >= 0).all() and (T <= 2 ** 32).all()
    vs, rs = [], []
    for x, t in zip(v, T):
        for r in (t - 1, t, 0, 2 ** 32 - 1):
            if 0 <= r < 2 ** 32:
                vs.append(x)
                rs.append(r)
    vs = np.array(vs, np.float32)
    rs = np.array(rs, np.uint64).astype(np.uint32)
    got = _device_sr(vs, rs)
    want = np.array([expected(x, int(r)) for x, r in zip(vs, rs)], np.uint8)
    bad = np.argwhere(got != want)
    assert len(bad) == 0, f"{len(bad)} differ; first v={vs[bad[0][0]]!r} r={rs[bad[0][0]]}: " \
                          f"{got[bad[0][0]]} vs {want[bad[0][0]]}"
    assert (R.sr_e2m1(vs, rs) == want).all()
    # at the threshold: r = T - 1 rounds up, r = T rounds down (off the grid)
    off = [i for i, x in enumerate(v) if threshold(x) not in (0,)]
    assert off, "no off-grid values"


def test_grid_values_never_move_and_saturation():
    mags = E2M1.magnitudes.astype(np.float32)
    v = np.concatenate([mags, -mags, np.float32([6.0, 7.0, 1e30, np.inf, -1e30, -np.inf])]).astype(np.float32)
    for r in (0, 1, 2 ** 31, 2 ** 32 - 1):
        got = _device_sr(v, np.full(len(v), r, np.uint32))
        want = np.array([expected(x, r) if np.isfinite(x) else (7 | (8 if x < 0 else 0)) for x in v], np.uint8)
        assert (got == want).all(), r


def test_nan_saturates_as_the_oracle_does():
    """A NaN (either sign bit) takes the largest magnitude, as in the oracle,
    whatever the random word."""
    v = np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFFFFFFFF], np.uint32).view(np.float32)
    for r in (0, 1, 2 ** 31, 2 ** 32 - 1):
        rs = np.full(len(v), r, np.uint32)
        got = _device_sr(v, rs)
        assert (got == R.sr_e2m1(v, rs)).all(), (r, got)
        assert (got & 7 == 7).all()


def test_empty_call_enqueues_nothing():
    P.pbs_debug_sr_encode(None, None, None, 0)
