"""Scaling recipes: amax, scale derivation, casts, RHT16 and stochastic rounding.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Conventions
-----------
* Inputs are 2-D arrays of bf16 bit patterns (uint16).  ``bf16_to_f32``
  turns them into exactly equal float32 values.
* Every floating-point step is one IEEE-754 binary32 operation done with
  NumPy float32 arithmetic (round-to-nearest-even), in exactly the order
  written; a chain such as fp32(fp32(a / 6) * S) is two roundings.
* A "row" copy quantizes along the stored columns of the input.  A "col"
  copy quantizes along the stored rows and is returned transposed, so that
  in both cases the quantization blocks run along the last (contiguous)
  axis of the returned array: the GEMM contraction axis.
* Any scale division that overflows float32 gives FLT_MAX; a zero amax gives
  scale 1 (per-tensor, sub-channel), E8M0 exponent -127 (MXFP8, MXFP4), or block
  scale 0 with +-0 codes (NVFP4).  The pages do not say what happens in
  these corner cases; this is the reading taken.
"""
from __future__ import annotations

import numpy as np

from .formats import E2M1, E4M3, E5M2, FORMATS, bf16_to_f32, e8m0_decode
from .philox import philox4x32_10, philox_word_for_index

FLT_MAX = np.float32(np.finfo(np.float32).max)
FMAX = {"e4m3": 448.0, "e5m2": 57344.0}
NVFP4_GLOBAL_NUMERATOR = 6.0 * 448.0          # E2M1 max times E4M3 max = 2688


def _f32(x):
    return np.asarray(x, dtype=np.float32)


def _oriented(x_bits, orient):
    """float32 values of ``x_bits`` with the quantization axis last."""
    t = bf16_to_f32(x_bits)
    if orient == "row":
        return t
    if orient == "col":
        return np.ascontiguousarray(t.T)
    raise ValueError(orient)


# ---------------------------------------------------------------------------
# amax and per-tensor scales
# ---------------------------------------------------------------------------
def amax(t):
    """max |t| over the tensor, exact (no rounding involved).

    "Optimizing Transformer models for low-precision training", "Technical
    deep-dive": the per-tensor scale maps the tensor's max absolute value to
    the FP8 range; "Faster training throughput in FP8 precision with NVIDIA
    NeMo", strengths and trade-offs, per-tensor current scaling item: the
    amax is taken in real time on the tensor about to be cast.
    """
    t = np.asarray(t)
    if t.dtype == np.uint16:
        t = bf16_to_f32(t)
    if t.size == 0:
        return np.float32(0.0)
    return np.float32(np.max(np.abs(t.astype(np.float32))))


def scale_from_amax(a, fmax):
    """s = fp32(fmax / a) (1 if a == 0, FLT_MAX on overflow); s_inv = fp32(1 / s).

    Works elementwise on arrays (sub-channel blocks) as well as scalars.
    """
    a = _f32(a)
    with np.errstate(divide="ignore", over="ignore"):
        s = np.float32(fmax) / np.where(a == 0, np.float32(1.0), a)
    s = np.where(a == 0, np.float32(1.0), s).astype(np.float32)
    s = np.where(np.isinf(s), FLT_MAX, s).astype(np.float32)
    s_inv = (np.float32(1.0) / s).astype(np.float32)
    return s, s_inv


# ---------------------------------------------------------------------------
# FP8 per-tensor current scaling
# ---------------------------------------------------------------------------
def cast_pertensor(x_bits, s, fmt, orient="row"):
    """q = enc_fmt(fp32(x * s)) for every element; ``s`` is the fp32 scale."""
    t = _oriented(x_bits, orient)
    v = (t * np.float32(s)).astype(np.float32)
    return FORMATS[fmt].encode(v)


def quantize_current(x_bits, fmt, orient="row"):
    """Per-tensor current scaling: amax -> scale -> cast, all on this tensor.

    Returns (codes, s_inv, amax).
    """
    a = amax(x_bits)
    s, s_inv = scale_from_amax(a, FMAX[fmt])
    return cast_pertensor(x_bits, s, fmt, orient), np.float32(s_inv), a


# ---------------------------------------------------------------------------
# FP8 per-tensor delayed scaling with an amax history
# ---------------------------------------------------------------------------
class DelayedScaling:
    """Scale taken from the maximum of a rolling window of past amax values.

    "Optimizing Transformer models for low-precision training", "Technical
    deep-dive": a rolling history of amax values is kept and the scale is
    computed from earlier iterations' statistics.  "Faster training
    throughput in FP8 precision with NVIDIA NeMo", per-tensor delayed
    scaling item: the scale comes from the history.

    Reading taken (the pages give no formula): history of ``hist_len``
    zeros, write position 0, scale 1 at start.  At step t the cast uses the
    current scale and the same pass measures amax_t; the GEMM of step t
    dequantizes with fp32(1/s).  Then amax_t is written at the write
    position, the position advances modulo ``hist_len``, and the new scale is
    fp32(fmax / max(history)) (1 if that max is 0, FLT_MAX on overflow).
    """

    def __init__(self, fmt, hist_len=16):
        self.fmt = fmt
        self.fmax = FMAX[fmt]
        self.hist = np.zeros(hist_len, dtype=np.float32)
        self.pos = 0
        self.scale = np.float32(1.0)

    def cast(self, x_bits, orient="row"):
        """Cast with the current scale.  Returns (codes, s_inv, amax_t)."""
        codes = cast_pertensor(x_bits, self.scale, self.fmt, orient)
        s_inv = np.float32(np.float32(1.0) / self.scale)
        return codes, s_inv, amax(x_bits)

    def update(self, amax_t):
        self.hist[self.pos] = np.float32(amax_t)
        self.pos = (self.pos + 1) % len(self.hist)
        s, _ = scale_from_amax(np.max(self.hist), self.fmax)
        self.scale = np.float32(s)

    def state_words(self):
        """(history, pos, scale, scale_inv) -- what one step leaves behind."""
        return (self.hist.copy(), self.pos, np.float32(self.scale),
                np.float32(np.float32(1.0) / self.scale))


# ---------------------------------------------------------------------------
# Sub-channel (generic block) FP8: 1x128 activations/gradients, 128x128 weights
# ---------------------------------------------------------------------------
def _block_amax(t, br, bc):
    r, c = t.shape
    if r % br or c % bc:
        raise ValueError("shape not a multiple of the block")
    return np.abs(t).reshape(r // br, br, c // bc, bc).max(axis=(1, 3)).astype(np.float32)


def _expand(s, br, bc):
    return np.repeat(np.repeat(s, br, axis=0), bc, axis=1)


def quantize_block128(x_bits, orient="row", weight_2d=False):
    """Sub-channel FP8 with fp32 block scales.

    "Faster training throughput in FP8 precision with NVIDIA NeMo",
    "Scaling recipe granularity": activations in 1x128 blocks and weights in
    128x128 blocks (the page's example; its label for it is garbled, and the
    pairings are read as (activations, weights) with 1D = 1x128 and 2D =
    128x128, so this is 1D2D; oracle.passes selects the shape per source for
    the 1D1D and 2D2D pairings); strengths and trade-offs, sub-channel item:
    configurable block dimensions, finer blocks cost more scale storage.
    Reading taken: per block, s_b = fp32(448 / amax_b) (same corner rules as
    the per-tensor scale), q = enc_E4M3(fp32(x * s_b)), and the stored scale
    is fp32(1 / s_b).  E4M3 for every role.

    Returns (codes [rows, cols], s_inv [rows, cols/128] or
    [rows/128, cols/128]) in the requested orientation.
    """
    t = _oriented(x_bits, orient)
    br, bc = (128, 128) if weight_2d else (1, 128)
    a_b = _block_amax(t, br, bc)
    s, s_inv = scale_from_amax(a_b, 448.0)
    v = (t * _expand(s, br, bc)).astype(np.float32)
    return E4M3.encode(v), s_inv


# ---------------------------------------------------------------------------
# Channel-wise FP8: one fp32 scale per row of the contraction-contiguous copy
# ---------------------------------------------------------------------------
def quantize_channel(x_bits, orient="row"):
    """Channel-wise FP8 (E4M3): one scale per row of the copy.

    "Faster training throughput in FP8 precision with NVIDIA NeMo",
    "Scaling recipe granularity": channel-wise scaling applies one factor per
    channel (row or column), a granularity between per-tensor and 2D blocks.
    Reading taken: one scale per row of the contraction-contiguous copy (the
    row copy: per row of x; the col copy: per column of x), computed like the
    sub-channel scales -- s_r = fp32(448 / amax_r) with the per-tensor corner
    rules, stored as fp32(1 / s_r); codes = enc_E4M3(fp32(x * s_r)).  In the
    GEMM both factors are constant along K, so C = acc * fp32(sa_inv[m] *
    sb_inv[n]).  Returns (codes [rows, cols], s_inv [rows]).
    """
    t = _oriented(x_bits, orient)
    a = np.max(np.abs(t), axis=1) if t.shape[1] else np.zeros(t.shape[0], np.float32)
    s, s_inv = scale_from_amax(a.astype(np.float32), 448.0)
    v = (t * s[:, None]).astype(np.float32)
    return E4M3.encode(v), s_inv.astype(np.float32)


# ---------------------------------------------------------------------------
# MXFP8: 32-value blocks, E8M0 power-of-two scales
# ---------------------------------------------------------------------------
_E8M0_THRESHOLDS = 448.0 * np.ldexp(1.0, np.arange(255) - 127)   # 448 * 2**e, e = -127..127


def mx_block_exponent_code(a_b):
    """E8M0 code c = e + 127 of the smallest e in [-127, 127] with a_b <= 448 * 2**e.

    "Faster training throughput in FP8 precision with NVIDIA NeMo",
    strengths and trade-offs, MXFP8 item: one power-of-two E8M0 scale per
    32-value block.  Reading taken for the exponent: the smallest power of
    two that brings the block maximum into the E4M3 range, so that no
    element saturates.  Found by searching all 255 finite E8M0 scales.
    """
    a = np.asarray(a_b, dtype=np.float64)
    return np.searchsorted(_E8M0_THRESHOLDS, a, side="left").astype(np.uint8)


def quantize_mxfp8(x_bits, orient="row"):
    """Returns (E4M3 codes [rows, cols], E8M0 codes [rows, cols/32])."""
    t = _oriented(x_bits, orient)
    a_b = _block_amax(t, 1, 32)
    c = mx_block_exponent_code(a_b)
    e = c.astype(np.int64) - 127
    v = t.astype(np.float64) * np.ldexp(1.0, -_expand(e, 1, 32))   # exact
    return E4M3.encode(v), c


def quantize_block128_pow2(x_bits, orient="row", weight_2d=False):
    """Sub-channel FP8 with power-of-two (E8M0) block scales.

    "Faster training throughput in FP8 precision with NVIDIA NeMo":
    "Scaling recipe granularity" sets the sub-channel blocks (1x128
    activations and gradients, 128x128 weights) and closes on the trade-off
    between granularity and throughput that hardware-native block scaling
    (MXFP8's E8M0 power-of-two scales, same page, strengths and trade-offs,
    MXFP8 item) avoids.  Reading taken for this variant: the sub-channel
    block shapes with MXFP8's scale rule -- per block, the smallest e in
    [-127, 127] with amax_b <= 448 * 2**e (stored as the E8M0 code e + 127),
    codes = enc_E4M3(x * 2**-e) (scaling by a power of two is exact, so only
    the encode rounds), x_hat = dec(q) * 2**e.  E4M3 for every role.

    Returns (codes [rows, cols], E8M0 codes [rows, cols/128] or
    [rows/128, cols/128]) in the requested orientation.
    """
    t = _oriented(x_bits, orient)
    br, bc = (128, 128) if weight_2d else (1, 128)
    c = mx_block_exponent_code(_block_amax(t, br, bc))
    e = c.astype(np.int64) - 127
    v = t.astype(np.float64) * np.ldexp(1.0, -_expand(e, br, bc))   # exact
    return E4M3.encode(v), c


# ---------------------------------------------------------------------------
# NVFP4: E2M1 values, E4M3 scale per 16 values, FP32 scale per tensor
# ---------------------------------------------------------------------------
def nvfp4_tensor_scales(global_amax):
    """S_enc = fp32(2688 / A) with the corner rules above; S_dec = fp32(1 / S_enc).

    "Accelerate LLM training with NVFP4 on Blackwell", "Technical
    deep-dive": a second-level FP32 scale covers the whole tensor.
    Reading taken: the tensor scale maps the tensor amax to the product of
    the E2M1 and E4M3 maxima, 6 * 448.
    """
    s, s_inv = scale_from_amax(global_amax, NVFP4_GLOBAL_NUMERATOR)
    return np.float32(s), np.float32(s_inv)


def sr_e2m1(v, r):
    """Stochastic rounding of fp32 values to E2M1 magnitudes with 32-bit randoms r.

    Reading taken: |v| >= 6 gives 6; otherwise, with lo <= |v| < hi the
    neighbouring E2M1 magnitudes, round up to hi iff r < P * 2**32 where
    P = (|v| - lo) / (hi - lo), compared exactly; the sign is kept.  Values
    on the grid never move and the expected result equals v.
    """
    v64 = np.asarray(v, dtype=np.float32).astype(np.float64)
    r64 = np.asarray(r, dtype=np.uint32).astype(np.float64)
    neg = np.signbit(v64)
    a = np.abs(v64)
    mags = E2M1.magnitudes
    lo_i = np.clip(np.searchsorted(mags, a, side="right") - 1, 0, len(mags) - 1)
    hi_i = np.minimum(lo_i + 1, len(mags) - 1)
    lo, hi = mags[lo_i], mags[hi_i]
    width = np.where(hi > lo, hi - lo, 1.0)
    threshold = (a - lo) / width * 4294967296.0          # exact dyadic value
    up = (r64 < threshold) & (hi > lo)
    code = np.where(up, hi_i, lo_i)
    code = np.where(a >= 6.0, 7, code)
    return (code | np.where(neg, 8, 0)).astype(np.uint8)


def pack_e2m1(codes):
    """Two E2M1 codes per byte along the last axis, even index in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    if codes.shape[-1] % 2:
        raise ValueError("odd length")
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def unpack_e2m1(packed):
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def quantize_nvfp4(t, S_enc, weight_2d=False, sr_random=None):
    """Two-level NVFP4 cast of fp32 values ``t`` (quantization axis last).

    "Accelerate LLM training with NVFP4 on Blackwell", "Technical
    deep-dive": E2M1 values, one E4M3 scale per 16-value micro-block, one
    FP32 scale per tensor.  "How to optimize Transformer-based models for
    low-precision training", "Interpreting results for a real model": 2D
    block scaling for weights, stochastic rounding for gradients.

    Reading taken, per block b (1x16 along the last axis, or 16x16 tiles for
    weights):
        a_b    = max |t| over the block
        d_code = enc_E4M3(fp32(fp32(a_b / 6) * S_enc)),  d = dec(d_code)
        if d == 0: every code is +-0 (sign of t)
        else: e_b = fp32(S_enc / d) (FLT_MAX on overflow), v = fp32(t * e_b),
              q = enc_E2M1(v), or SR(v) when ``sr_random`` (uint32, same shape
              as t) is given.
    Returns (packed codes [rows, cols/2], d_codes).
    """
    t = _f32(t)
    br, bc = (16, 16) if weight_2d else (1, 16)
    a_b = _block_amax(t, br, bc)
    d_val = ((a_b / np.float32(6.0)).astype(np.float32) * np.float32(S_enc)).astype(np.float32)
    d_code = E4M3.encode(d_val)
    d = E4M3.decode(d_code).astype(np.float32)
    with np.errstate(divide="ignore", over="ignore"):
        e_b = (np.float32(S_enc) / np.where(d == 0, np.float32(1.0), d)).astype(np.float32)
    e_b = np.where(np.isinf(e_b), FLT_MAX, e_b).astype(np.float32)
    v = (t * _expand(e_b, br, bc)).astype(np.float32)
    if sr_random is None:
        q = E2M1.encode(v)
    else:
        q = sr_e2m1(v, sr_random)
    zero_block = _expand(d == 0, br, bc)
    q = np.where(zero_block, np.where(np.signbit(t), 8, 0), q).astype(np.uint8)
    return pack_e2m1(q), d_code


def sr_random_for(shape_mn, orient, seed=42):
    """Per-element SR random words for a gradient dY of logical shape [M, N].

    Element (m, n) takes word i % 4 of the Philox call with counter i // 4,
    i = m * N + n its logical index in dY, whatever copy is being produced;
    returned in the layout of the requested copy.
    """
    M, N = shape_mn
    idx = np.arange(M * N, dtype=np.uint64).reshape(M, N)
    r = philox_word_for_index(idx, seed)
    return r if orient == "row" else np.ascontiguousarray(r.T)


# ---------------------------------------------------------------------------
# MXFP4: E2M1 values, E8M0 power-of-two scale per 32 values
# ---------------------------------------------------------------------------
_E8M0_THRESHOLDS_FP4 = 6.0 * np.ldexp(1.0, np.arange(255) - 127)   # 6 * 2**e, e = -127..127


def mx4_block_exponent_code(a_b):
    """E8M0 code c = e + 127 of the smallest e in [-127, 127] with a_b <= 6 * 2**e.

    "Accelerate LLM training with NVFP4 on Blackwell", "Technical
    deep-dive": NVFP4's 16-value micro-blocks are a reduction from MXFP4's
    32.  MXFP4 keeps the MX scale (one E8M0 power of two per block, as for
    MXFP8) over E2M1 values.  Reading taken for the exponent, the same as
    for MXFP8 with E2M1's maximum 6: the smallest power of two that brings
    the block maximum into range, so that no element saturates.
    """
    a = np.asarray(a_b, dtype=np.float64)
    return np.searchsorted(_E8M0_THRESHOLDS_FP4, a, side="left").astype(np.uint8)


def quantize_mxfp4(t, sr_random=None):
    """MXFP4 cast of fp32 values ``t`` (quantization axis last, 1x32 blocks).

    Per block b: c = mx4_block_exponent_code(max |t|), e = c - 127,
    v = fp32(t * 2**-e), q = enc_E2M1(v) (round to nearest even), or the
    stochastic rounding of v when ``sr_random`` (uint32, same shape as t)
    is given.  A zero block gets c = 0 and +-0 codes.
    Returns (packed codes [rows, cols/2], E8M0 codes [rows, cols/32]).
    """
    t = _f32(t)
    a_b = _block_amax(t, 1, 32)
    c = mx4_block_exponent_code(a_b)
    e = c.astype(np.int64) - 127
    v = (t.astype(np.float64) * np.ldexp(1.0, -_expand(e, 1, 32))).astype(np.float32)
    q = E2M1.encode(v) if sr_random is None else sr_e2m1(v, sr_random)
    return pack_e2m1(q), c


# ---------------------------------------------------------------------------
# Random Hadamard transform, 16x16
# ---------------------------------------------------------------------------
def rht_signs(seed=42):
    """sigma_j = +1 if bit 0 of word 0 of Philox(key=(seed,0), ctr=(j,0,1,0)) is 0, else -1."""
    w0 = philox4x32_10(np.arange(16, dtype=np.uint64), 0, 1, 0,
                       seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)[0]
    return np.where((w0 & 1) == 0, 1.0, -1.0).astype(np.float32)


def rht16_along_rows(t, seed=42):
    """y = 1/4 * H16 * D * x on every group of 16 consecutive rows of each column.

    "How to optimize Transformer-based models for low-precision training",
    "Using autocast mode vs pre-quantized mode" and "Interpreting results
    for a real model": a random Hadamard transform is applied to the Wgrad
    inputs.  Reading taken: Sylvester-ordered H16, random signs D from
    ``rht_signs``, normalisation 1/4 so the transform is orthogonal, applied
    along the token axis M (the Wgrad contraction axis) in four butterfly
    stages (h = 1, 2, 4, 8), each a float32 add and subtract, then an exact
    float32 multiply by 0.25.  The result stays float32.
    """
    t = _f32(t)
    M, C = t.shape
    if M % 16:
        raise ValueError("rows not a multiple of 16")
    sig = rht_signs(seed)
    u = [(t[j::16, :] * sig[j]).astype(np.float32) for j in range(16)]
    for h in (1, 2, 4, 8):
        for i in range(16):
            if i & h == 0:
                a, b = u[i], u[i + h]
                u[i], u[i + h] = (a + b).astype(np.float32), (a - b).astype(np.float32)
    y = np.empty_like(t)
    for j in range(16):
        y[j::16, :] = (u[j] * np.float32(0.25)).astype(np.float32)
    return y


# ---------------------------------------------------------------------------
# Dequantization (exact, float64) -- the operands the reference GEMM consumes
# ---------------------------------------------------------------------------
def dequant_pertensor(codes, fmt, s_inv):
    return FORMATS[fmt].decode(codes) * np.float64(np.float32(s_inv))


def dequant_block128(codes, s_inv, weight_2d=False):
    br, bc = (128, 128) if weight_2d else (1, 128)
    return E4M3.decode(codes) * _expand(np.asarray(s_inv, dtype=np.float32).astype(np.float64), br, bc)


def dequant_channel(codes, s_inv):
    return E4M3.decode(codes) * np.asarray(s_inv, np.float32).astype(np.float64)[:, None]


def dequant_mxfp8(codes, e8m0_codes):
    return E4M3.decode(codes) * _expand(e8m0_decode(e8m0_codes), 1, 32)


def dequant_block128_pow2(codes, e8m0_codes, weight_2d=False):
    br, bc = (128, 128) if weight_2d else (1, 128)
    return E4M3.decode(codes) * _expand(e8m0_decode(e8m0_codes), br, bc)


def dequant_mxfp4(packed, e8m0_codes):
    return E2M1.decode(unpack_e2m1(packed)) * _expand(e8m0_decode(e8m0_codes), 1, 32)


def dequant_nvfp4(packed, d_codes, S_dec, weight_2d=False):
    br, bc = (16, 16) if weight_2d else (1, 16)
    q = E2M1.decode(unpack_e2m1(packed))
    d = E4M3.decode(d_codes)
    return q * _expand(d, br, bc) * np.float64(np.float32(S_dec))
