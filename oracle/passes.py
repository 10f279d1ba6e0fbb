"""Which quantized copy each GEMM consumes, per recipe and pass.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"How to optimize Transformer-based models for low-precision training",
"Using autocast mode vs pre-quantized mode": Fprop, Dgrad and Wgrad are
separate GEMMs.  With X [M, K] (activations), W [N, K] (weights, stored
output-major) and dY [M, N] (output gradient):

  Fprop  Y  = X  . W^T   contraction K:  A = X  (blocks along K),  B = W  (along K)
  Dgrad  dX = dY . W     contraction N:  A = dY (along N),         B = W^T (along N)
  Wgrad  dW = X^T . dY   contraction M:  A = X^T (along M),        B = dY^T (along M)

Both operands are produced with the contraction axis last.  Format roles
(reading taken from "Optimizing Transformer models for low-precision
training", "Technical deep-dive": E4M3 for forward activations and weights,
E5M2 for gradients): per-tensor recipes use E4M3 for X and W and E5M2 for
dY; sub-channel and MXFP8 use E4M3 for every role; NVFP4 uses E2M1.
Weights take 2D blocks (128x128 sub-channel, 16x16 NVFP4).  NVFP4 applies
the 16x16 random Hadamard transform to both Wgrad operands (along M) and
stochastic rounding to dY (both copies); everything else rounds to nearest.

MXFP4 ("Accelerate LLM training with NVFP4 on Blackwell", "Technical
deep-dive": the 32-value format NVFP4 refines) is built as the next recipe
after the pages' six.  Reading taken: E2M1 values with one E8M0 scale per
1x32 block along the contraction axis for every operand (each orientation
quantized from the source, as MXFP8 does), and NVFP4's 4-bit training
treatment kept: the Hadamard transform on both Wgrad operands and
stochastic rounding of dY.

Channel-wise FP8 ("Faster training throughput in FP8 precision with NVIDIA
NeMo", "Scaling recipe granularity": one factor per channel, between
per-tensor and 2D blocks) is the other next recipe: E4M3 for every role, one
fp32 scale per row of each contraction-contiguous copy.

The other sub-channel block pairings (same page, same section: "1D1D" and
"1D2D" beside the 1x128-activation / 128x128-weight example) are read as
naming the block shape of (activations and gradients, weights), 1D = 1x128
and 2D = 128x128: the recipe above is 1D2D; "fp8_block128_1d1d" gives every
tensor 1x128 blocks along the contraction axis (the weight's col copy is
quantized from the source, not transposed), "fp8_block128_2d2d" gives every
tensor 128x128 blocks (each col copy is the transposed row copy).

"fp8_block128_pow2" keeps the 1D2D block shapes (1x128 activations and
gradients, 128x128 weights) and takes MXFP8's power-of-two scale rule per
block instead of the fp32 scale: the sub-channel granularity with
hardware-native (E8M0) block scales, which the same section sets against
generic block scaling.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import recipes as R
from .formats import bf16_to_f32

RECIPES = ("bf16", "fp8_current", "fp8_delayed", "fp8_block128", "mxfp8", "nvfp4")
# sub-channel recipes -> the sources that take 128x128 blocks (the rest 1x128)
BLOCK128_2D = {"fp8_block128": ("w",), "fp8_block128_1d1d": (), "fp8_block128_2d2d": ("x", "w", "dy")}
NEXT_RECIPES = ("mxfp4", "fp8_channel", "fp8_block128_1d1d", "fp8_block128_2d2d", "fp8_block128_pow2")
ALL_RECIPES = RECIPES + NEXT_RECIPES


@dataclass
class QOperand:
    """A quantized GEMM operand, contraction axis last."""
    recipe: str
    fmt: str
    codes: np.ndarray                  # uint8 codes (E2M1 packed 2 per byte), or bf16 bits
    scale: np.ndarray | None = None    # block scales (fp32 s_inv / E8M0 codes / E4M3 codes)
    tensor_scale_inv: np.float32 | None = None
    weight_2d: bool = False
    extra: dict = field(default_factory=dict)

    def dequant(self):
        if self.recipe == "bf16":
            return bf16_to_f32(self.codes).astype(np.float64)
        if self.recipe in ("fp8_current", "fp8_delayed"):
            return R.dequant_pertensor(self.codes, self.fmt, self.tensor_scale_inv)
        if self.recipe in BLOCK128_2D:
            return R.dequant_block128(self.codes, self.scale, self.weight_2d)
        if self.recipe == "fp8_block128_pow2":
            return R.dequant_block128_pow2(self.codes, self.scale, self.weight_2d)
        if self.recipe == "mxfp8":
            return R.dequant_mxfp8(self.codes, self.scale)
        if self.recipe == "nvfp4":
            return R.dequant_nvfp4(self.codes, self.scale, self.tensor_scale_inv, self.weight_2d)
        if self.recipe == "mxfp4":
            return R.dequant_mxfp4(self.codes, self.scale)
        if self.recipe == "fp8_channel":
            return R.dequant_channel(self.codes, self.scale)
        raise ValueError(self.recipe)


def operand_roles(pass_):
    """(A source, A orient), (B source, B orient) for a pass."""
    return {"fprop": (("x", "row"), ("w", "row")),
            "dgrad": (("dy", "row"), ("w", "col")),
            "wgrad": (("x", "col"), ("dy", "col"))}[pass_]


def _pertensor_fmt(src):
    return "e5m2" if src == "dy" else "e4m3"


def quantize_operand(recipe, src, orient, x_bits, pass_, delayed_state=None, seed=42):
    """Quantize one source tensor ('x', 'w' or 'dy') for use in ``pass_``."""
    if recipe == "bf16":
        t = x_bits if orient == "row" else np.ascontiguousarray(x_bits.T)
        return QOperand("bf16", "bf16", t)
    if recipe == "fp8_current":
        fmt = _pertensor_fmt(src)
        codes, s_inv, a = R.quantize_current(x_bits, fmt, orient)
        return QOperand(recipe, fmt, codes, tensor_scale_inv=s_inv, extra={"amax": a})
    if recipe == "fp8_delayed":
        if delayed_state is None:
            raise ValueError("delayed scaling needs its state")
        codes, s_inv, a = delayed_state.cast(x_bits, orient)
        return QOperand(recipe, delayed_state.fmt, codes, tensor_scale_inv=s_inv,
                        extra={"amax": a})
    if recipe in BLOCK128_2D:
        w2d = src in BLOCK128_2D[recipe]
        codes, s_inv = R.quantize_block128(x_bits, orient, weight_2d=w2d)
        return QOperand(recipe, "e4m3", codes, scale=s_inv, weight_2d=w2d)
    if recipe == "fp8_block128_pow2":
        w2d = src == "w"
        codes, e8 = R.quantize_block128_pow2(x_bits, orient, weight_2d=w2d)
        return QOperand(recipe, "e4m3", codes, scale=e8, weight_2d=w2d)
    if recipe == "mxfp8":
        codes, e8 = R.quantize_mxfp8(x_bits, orient)
        return QOperand(recipe, "e4m3", codes, scale=e8)
    if recipe == "nvfp4":
        w2d = src == "w"
        t = bf16_to_f32(x_bits)
        rht = pass_ == "wgrad"
        if rht:
            t = R.rht16_along_rows(t, seed)
        A = R.amax(t)
        S_enc, S_dec = R.nvfp4_tensor_scales(A)
        t_o = t if orient == "row" else np.ascontiguousarray(t.T)
        sr = None
        if src == "dy":
            sr = R.sr_random_for(x_bits.shape, orient, seed)
        packed, d_codes = R.quantize_nvfp4(t_o, S_enc, weight_2d=w2d, sr_random=sr)
        return QOperand(recipe, "e2m1", packed, scale=d_codes, tensor_scale_inv=S_dec,
                        weight_2d=w2d, extra={"amax": A, "S_enc": S_enc, "rht": rht,
                                              "sr": sr is not None})
    if recipe == "fp8_channel":
        codes, s_inv = R.quantize_channel(x_bits, orient)
        return QOperand(recipe, "e4m3", codes, scale=s_inv)
    if recipe == "mxfp4":
        t = bf16_to_f32(x_bits)
        rht = pass_ == "wgrad"
        if rht:
            t = R.rht16_along_rows(t, seed)
        t_o = t if orient == "row" else np.ascontiguousarray(t.T)
        sr = R.sr_random_for(x_bits.shape, orient, seed) if src == "dy" else None
        packed, e8 = R.quantize_mxfp4(t_o, sr_random=sr)
        return QOperand(recipe, "e2m1", packed, scale=e8,
                        extra={"rht": rht, "sr": sr is not None})
    raise ValueError(recipe)


def pass_operands(recipe, pass_, x=None, w=None, dy=None, delayed_states=None, seed=42):
    """Quantized (A, B) for one GEMM.  ``delayed_states`` maps 'x'/'w'/'dy' to states."""
    srcs = {"x": x, "w": w, "dy": dy}
    (sa, oa), (sb, ob) = operand_roles(pass_)
    st = delayed_states or {}
    a = quantize_operand(recipe, sa, oa, srcs[sa], pass_, st.get(sa), seed)
    b = quantize_operand(recipe, sb, ob, srcs[sb], pass_, st.get(sb), seed)
    return a, b
