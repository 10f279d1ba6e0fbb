"""Pins for the oracle's codecs (CPU only).

Each check compares the oracle's table-search codec with something other
than itself: PyTorch's float8 dtypes (a library routine), exact rational
arithmetic, the bit splits and value range the pages print, or brute force.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle.formats import E2M1, E4M3, E5M2, e8m0_decode, bf16_to_f32, f32_to_bf16_rne

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


def _torch_decode(codes, dtype):
    t = torch.tensor(np.asarray(codes, dtype=np.uint8)).view(dtype)
    return t.to(torch.float32).numpy().astype(np.float64)


@pytest.mark.parametrize("fmt,dtype", [(E4M3, torch.float8_e4m3fn), (E5M2, torch.float8_e5m2)])
def test_fp8_decode_all_256_codes_match_torch(fmt, dtype):
    codes = np.arange(256)
    ours = fmt.decode(codes)
    ref = _torch_decode(codes, dtype)
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()
    # signed zero too
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0])


def test_bit_splits_and_maxima_match_pages():
    g = GOLDEN["fp8_bit_splits"]
    assert (E4M3.ebits, E4M3.mbits) == (g["e4m3"]["exponent"], g["e4m3"]["mantissa"])
    assert (E5M2.ebits, E5M2.mbits) == (g["e5m2"]["exponent"], g["e5m2"]["mantissa"])
    n = GOLDEN["nvfp4"]
    assert (E2M1.ebits, E2M1.mbits) == (n["e2m1"]["exponent"], n["e2m1"]["mantissa"])
    assert E2M1.max_value == n["value_range_abs"]
    assert E4M3.max_value == 448.0 and E5M2.max_value == 57344.0


def test_e2m1_all_16_codes():
    vals = E2M1.decode(np.arange(16))
    assert list(vals[:8]) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(vals[8:]) == [-0.0, -0.5, -1, -1.5, -2, -3, -4, -6]
    assert np.signbit(vals[8])


def test_e2m1_ties_and_saturation():
    # ties go to the even code (mantissa bit 0)
    cases = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0,
             6.5: 6.0, 100.0: 6.0, 0.2: 0.0, 0.3: 0.5, 2.6: 3.0, 5.1: 6.0}
    for v, want in cases.items():
        assert E2M1.decode(E2M1.encode(np.float32(v)))[()] == want, v
        assert E2M1.decode(E2M1.encode(np.float32(-v)))[()] == -want, v


def test_e8m0_all_codes_match_torch():
    codes = np.arange(256)
    ours = e8m0_decode(codes)
    ref = _torch_decode(codes, torch.float8_e8m0fnu)
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert (ours[:255] == ref[:255]).all()
    assert ours[127] == 1.0


@pytest.mark.parametrize("fmt", [E4M3, E5M2, E2M1])
def test_roundtrip_every_finite_code(fmt):
    codes = np.arange(fmt.max_code + 1)
    for sign in (0, fmt.sign_bit):
        c = codes | sign
        assert (fmt.encode(fmt.decode(c).astype(np.float32)) == c).all()


@pytest.mark.parametrize("fmt", [E4M3, E5M2, E2M1])
def test_midpoints_go_to_even_and_neighbours_to_nearest(fmt):
    m = fmt.magnitudes
    mids = ((m[:-1] + m[1:]) / 2).astype(np.float32)
    assert (mids.astype(np.float64) == (m[:-1] + m[1:]) / 2).all()   # exact in fp32
    got = fmt.encode(mids).astype(np.int64)
    lo = np.arange(len(m) - 1)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert (got == want).all()
    below = np.nextafter(mids, np.float32(-np.inf))
    above = np.nextafter(mids, np.float32(np.inf))
    assert (fmt.encode(below).astype(np.int64) == lo).all()
    assert (fmt.encode(above).astype(np.int64) == lo + 1).all()


@pytest.mark.parametrize("fmt", [E4M3, E5M2, E2M1])
def test_saturation_and_underflow(fmt):
    big = np.array([fmt.max_value * 1.01, fmt.max_value * 1e6, 3e38], dtype=np.float32)
    assert (fmt.encode(big) == fmt.max_code).all()
    assert (fmt.encode(-big) == (fmt.max_code | fmt.sign_bit)).all()
    half_min = np.float32(fmt.magnitudes[1] / 2)
    tiny = np.array([half_min, np.nextafter(half_min, np.float32(0)), 1e-30, 0.0], dtype=np.float32)
    assert (fmt.encode(tiny) == 0).all()
    assert (fmt.encode(-tiny) == fmt.sign_bit).all()
    assert fmt.encode(np.nextafter(half_min, np.float32(1)))[()] == 1


@pytest.mark.parametrize("fmt,dtype", [(E4M3, torch.float8_e4m3fn), (E5M2, torch.float8_e5m2)])
def test_encode_matches_torch_in_range(fmt, dtype):
    # every bf16 pattern, scaled into the format's range by several factors,
    # plus random fp32 values; torch rounds to nearest-even but does not
    # saturate, so only |v| <= max is compared.
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bf16_to_f32(b)
    rng = np.random.default_rng(5)
    vals = [x, rng.standard_normal(200000).astype(np.float32) * np.float32(fmt.max_value / 4)]
    for f in (np.float32(2.0 ** -100), np.float32(1e-3), np.float32(3.0)):
        vals.append((x * f).astype(np.float32))
    v = np.concatenate(vals)
    v = v[np.isfinite(v) & (np.abs(v) <= fmt.max_value)]
    ours = fmt.encode(v)
    ref = torch.from_numpy(v).to(dtype).view(torch.uint8).numpy()
    assert (ours == ref).all()


def _fraction_nearest_code(fmt, v):
    """Brute force: exact rational distance to every finite magnitude."""
    a = abs(Fraction(float(v)))
    if a > Fraction(fmt.max_value):
        code = fmt.max_code
    else:
        best = None
        for c, m in enumerate(fmt.magnitudes):
            d = abs(a - Fraction(float(m)))
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                best = (d, c)
        code = best[1]
    return code | (fmt.sign_bit if np.signbit(v) else 0)


@pytest.mark.parametrize("fmt", [E4M3, E5M2, E2M1])
def test_encode_matches_bruteforce_fraction(fmt):
    rng = np.random.default_rng(11)
    v = np.concatenate([
        rng.standard_normal(300).astype(np.float32) * np.float32(fmt.max_value / 3),
        (rng.standard_normal(300) * 1e-3).astype(np.float32) * np.float32(fmt.magnitudes[1] * 1e3),
        np.array([0.0, -0.0, fmt.max_value, -fmt.max_value * 2], dtype=np.float32)])
    ours = fmt.encode(v)
    for vi, oi in zip(v, ours):
        assert oi == _fraction_nearest_code(fmt, vi), (vi, oi)


def test_f32_to_bf16_rne_matches_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 1e3,
                        (rng.standard_normal(1000) * 1e-39).astype(np.float32)])
    ours = f32_to_bf16_rne(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == ref).all()
