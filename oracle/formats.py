"""Minifloat and scale formats, encoded by searching a table of magnitudes.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Formats (bit splits from "Optimizing Transformer models for low-precision
training", "Technical deep-dive", for E4M3 / E5M2; from "Accelerate LLM
training with NVFP4 on Blackwell", "Technical deep-dive", for E2M1 with
range about +-6; E8M0 power-of-two scales from "Faster training throughput
in FP8 precision with NVIDIA NeMo", "What are the strengths and trade-offs
of the FP8 scaling recipes?", MXFP8 item):

  E4M3 (OCP "FN" variant): sign, 4 exponent bits (bias 7), 3 mantissa bits.
       Largest finite magnitude 448 (code 0x7E); code 0x7F is NaN; no Inf.
  E5M2: sign, 5 exponent bits (bias 15), 2 mantissa bits.  Largest finite
       57344 (0x7B); exponent field 31 is Inf / NaN.
  E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit.  Magnitudes
       0, 0.5, 1, 1.5, 2, 3, 4, 6.  No specials.
  E8M0: 8-bit unsigned biased exponent, value 2**(c-127); 0xFF is NaN.

Reading taken where the pages are silent: encoding is round-to-nearest,
ties to the code whose mantissa LSB is 0, with saturation (a magnitude above
the largest finite value encodes to that value, with its sign), and the
sign of zero is kept.

The encoder never manipulates bits of the input: it looks the magnitude up
in the sorted list of every finite value the format can hold (built from the
bit definition above) and takes the nearest entry.  Within each format the
positive codes 0..max_code enumerate the magnitudes in increasing order, so
"mantissa LSB is 0" is "the code is even".
"""
from __future__ import annotations

import numpy as np


class MiniFloat:
    """A sign / exponent / mantissa format with no implicit NaN handling."""

    def __init__(self, name, ebits, mbits, bias, max_code, nan_codes=(), inf_codes=()):
        self.name = name
        self.ebits = ebits
        self.mbits = mbits
        self.bias = bias
        self.max_code = max_code          # largest finite positive code
        self.sign_bit = 1 << (ebits + mbits)
        self.nan_codes = set(nan_codes)
        self.inf_codes = set(inf_codes)
        mags = [self._value_of_positive_code(c) for c in range(max_code + 1)]
        self.magnitudes = np.array(mags, dtype=np.float64)
        assert np.all(np.diff(self.magnitudes) > 0), "codes must enumerate increasing values"
        self.max_value = float(self.magnitudes[-1])

    def _value_of_positive_code(self, c):
        e = c >> self.mbits
        f = c & ((1 << self.mbits) - 1)
        if e == 0:                                   # subnormal: f * 2**(1-bias-mbits)
            return f * 2.0 ** (1 - self.bias - self.mbits)
        return (1.0 + f / (1 << self.mbits)) * 2.0 ** (e - self.bias)

    # -- decode ---------------------------------------------------------
    def decode(self, codes):
        """Exact value of each code, as float64 (NaN / +-Inf for specials)."""
        codes = np.asarray(codes).astype(np.int64)
        mag_code = codes & (self.sign_bit - 1)
        neg = (codes & self.sign_bit) != 0
        out = np.empty(codes.shape, dtype=np.float64)
        finite = mag_code <= self.max_code
        out[finite] = self.magnitudes[mag_code[finite]]
        special = ~finite
        if np.any(special):
            vals = np.full(int(special.sum()), np.nan)
            sc = mag_code[special]
            for ic in self.inf_codes:
                vals[sc == ic] = np.inf
            out[special] = vals
        return np.where(neg, -out, out)

    # -- encode ---------------------------------------------------------
    def encode(self, v):
        """Round-to-nearest-even, saturating encode of the values ``v``.

        ``v`` is any float array (float32 values are represented exactly in
        float64).  An infinite value -- a scaled fp32 product that overflowed,
        whose exact magnitude is above every finite code -- saturates like
        any other value above the maximum.  Returns uint8 codes.
        """
        v = np.asarray(v)
        if np.any(np.isnan(v)):
            raise ValueError("NaN input is outside the encoder's contract")
        v64 = v.astype(np.float64)     # +-Inf (a scaled value that overflowed fp32) saturates
        neg = np.signbit(v64)
        a = np.abs(v64)
        mags = self.magnitudes
        idx = np.searchsorted(mags, np.minimum(a, self.max_value), side="left")
        hi = np.minimum(idx, len(mags) - 1)
        lo = np.maximum(hi - 1, 0)
        d_hi = mags[hi] - a
        d_lo = a - mags[lo]
        pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
        code = np.where(pick_hi, hi, lo)
        code = np.where(mags[hi] == a, hi, code)          # exact hit
        code = np.where(a > self.max_value, self.max_code, code)   # saturate
        code = code.astype(np.int64) | np.where(neg, self.sign_bit, 0)
        return code.astype(np.uint8)


E4M3 = MiniFloat("e4m3", ebits=4, mbits=3, bias=7, max_code=0x7E, nan_codes=(0x7F,))
E5M2 = MiniFloat("e5m2", ebits=5, mbits=2, bias=15, max_code=0x7B,
                 nan_codes=(0x7D, 0x7E, 0x7F), inf_codes=(0x7C,))
E2M1 = MiniFloat("e2m1", ebits=2, mbits=1, bias=1, max_code=0x7)

FORMATS = {"e4m3": E4M3, "e5m2": E5M2, "e2m1": E2M1}


def e8m0_decode(codes):
    """E8M0 scale value 2**(c-127) as float64; code 0xFF is NaN."""
    c = np.asarray(codes).astype(np.int64)
    out = np.ldexp(1.0, c - 127).astype(np.float64)
    return np.where(c == 255, np.nan, out)


def bf16_to_f32(bits):
    """bf16 bit patterns (uint16) -> exactly equal float32 values."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_rne(x):
    """float32 -> bf16 bit patterns, round-to-nearest-even (finite inputs).

    Used only to produce bf16 GEMM outputs for comparison; the rounding is
    done on the exact float64 value by table-free arithmetic: the candidate
    neighbours are the truncation and the truncation plus one unit.
    """
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    trunc = (u >> 16).astype(np.uint64)
    lo_val = (trunc << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    hi_val = ((trunc + 1) << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    xv = x.astype(np.float64)
    d_lo = np.abs(xv - lo_val)
    d_hi = np.abs(hi_val - xv)
    up = (d_hi < d_lo) | ((d_hi == d_lo) & ((trunc & 1) == 1))
    return np.where(up, trunc + 1, trunc).astype(np.uint16)
