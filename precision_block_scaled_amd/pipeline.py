"""Quantize-then-GEMM for one linear-layer GEMM, on top of the C ABI.

Buffer management and call sequencing only (torch allocates device memory,
every computation is a libpbs kernel).  Which copy each GEMM consumes
("How to optimize Transformer-based models for low-precision training",
"Using autocast mode vs pre-quantized mode": Fprop, Dgrad and Wgrad are
separate GEMMs), with X [M, K], W stored [N, K], dY [M, N]:

  fprop: A = X row copy,  B = W row copy
  dgrad: A = dY row copy, B = W col copy
  wgrad: A = X col copy,  B = dY col copy

Format roles: per-tensor FP8 uses E4M3 for X and W, E5M2 for dY;
sub-channel FP8 (fp32 or power-of-two block scales), channel-wise FP8 (one
fp32 scale per row of each copy) and MXFP8 use E4M3; NVFP4 and MXFP4 use E2M1.  Weights
take 2D blocks (128x128 sub-channel, 16x16 NVFP4; MXFP4 keeps 1x32 blocks
along the contraction axis for every operand); the sub-channel pairings
take 1x128 blocks on every tensor (1D1D) or 128x128 on every tensor (2D2D).  NVFP4 and MXFP4 apply the
random Hadamard transform to both Wgrad operands and stochastic rounding
to dY.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import (PBS_COL, PBS_DGRAD, PBS_FLAG_RHT16, PBS_FLAG_SR, PBS_FMT_BF16, PBS_FMT_E2M1,
               PBS_FMT_E4M3, PBS_FMT_E5M2, PBS_FMT_F32, PBS_FPROP, PBS_RECIPE_BF16,
               PBS_RECIPE_FP8_BLOCK128, PBS_RECIPE_FP8_BLOCK128_1D1D, PBS_RECIPE_FP8_BLOCK128_2D2D,
               PBS_RECIPE_FP8_BLOCK128_POW2,
               PBS_RECIPE_FP8_CHANNEL, PBS_RECIPE_FP8_CURRENT,
               PBS_RECIPE_FP8_DELAYED,
               PBS_RECIPE_MXFP4, PBS_RECIPE_MXFP8, PBS_RECIPE_NVFP4, PBS_ROW, PBS_WGRAD, pbs_amax,
               pbs_cast,
               pbs_delayed_init, pbs_delayed_scale, pbs_delayed_scale_inv, pbs_delayed_state_bytes,
               pbs_delayed_update, pbs_gemm, pbs_gemm_amax, pbs_scale_from_amax)

RECIPES = {
    "bf16": PBS_RECIPE_BF16,
    "fp8_current": PBS_RECIPE_FP8_CURRENT,
    "fp8_delayed": PBS_RECIPE_FP8_DELAYED,
    "fp8_block128": PBS_RECIPE_FP8_BLOCK128,
    "mxfp8": PBS_RECIPE_MXFP8,
    "nvfp4": PBS_RECIPE_NVFP4,
    "mxfp4": PBS_RECIPE_MXFP4,
    "fp8_channel": PBS_RECIPE_FP8_CHANNEL,
    "fp8_block128_1d1d": PBS_RECIPE_FP8_BLOCK128_1D1D,
    "fp8_block128_2d2d": PBS_RECIPE_FP8_BLOCK128_2D2D,
    "fp8_block128_pow2": PBS_RECIPE_FP8_BLOCK128_POW2,
}
# sources that take 2D blocks, per recipe
TWO_D = {"fp8_block128": ("w",), "nvfp4": ("w",), "fp8_block128_2d2d": ("x", "w", "dy"),
         "fp8_block128_pow2": ("w",)}
SUBCHANNEL = ("fp8_block128", "fp8_block128_1d1d", "fp8_block128_2d2d")
LAYOUTS = {"fprop": PBS_FPROP, "dgrad": PBS_DGRAD, "wgrad": PBS_WGRAD}
ROLES = {"fprop": (("x", "row"), ("w", "row")),
         "dgrad": (("dy", "row"), ("w", "col")),
         "wgrad": (("x", "col"), ("dy", "col"))}
FMAX = {PBS_FMT_E4M3: 448.0, PBS_FMT_E5M2: 57344.0}
NVFP4_FMAX = 2688.0
RHT_SEED = 42
SR_SEED = 42
HIST_LEN = 16


@dataclass
class QTensor:
    """One quantized copy, contraction axis last: codes [rows, cols(/2)]."""
    recipe: str
    fmt: int
    rows: int
    cols: int
    codes: torch.Tensor
    scales: torch.Tensor | None = None
    tensor_scale_inv: torch.Tensor | None = None
    weight_2d: bool = False


def fmt_for(recipe, src):
    if recipe in ("fp8_current", "fp8_delayed"):
        return PBS_FMT_E5M2 if src == "dy" else PBS_FMT_E4M3
    if recipe in ("nvfp4", "mxfp4"):
        return PBS_FMT_E2M1
    if recipe == "bf16":
        return PBS_FMT_BF16
    return PBS_FMT_E4M3


def _empty_copy(recipe, rows, cols, w2d, device):
    """Allocate codes / scales for one copy of stored shape [rows, cols]."""
    if recipe == "nvfp4":
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=device)
        sc = (torch.empty((rows // 16, cols // 16), dtype=torch.uint8, device=device) if w2d
              else torch.empty((rows, cols // 16), dtype=torch.uint8, device=device))
        return codes, sc
    if recipe == "mxfp4":
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=device)
        return codes, torch.empty((rows, cols // 32), dtype=torch.uint8, device=device)
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=device)
    if recipe == "fp8_block128_pow2":      # one 32-bit word per block: its E8M0 code in every byte
        sc = (torch.empty((rows // 128, cols // 128), dtype=torch.int32, device=device) if w2d
              else torch.empty((rows, cols // 128), dtype=torch.int32, device=device))
    elif recipe in SUBCHANNEL:
        sc = (torch.empty((rows // 128, cols // 128), dtype=torch.float32, device=device) if w2d
              else torch.empty((rows, cols // 128), dtype=torch.float32, device=device))
    elif recipe == "mxfp8":
        sc = torch.empty((rows, cols // 32), dtype=torch.uint8, device=device)
    elif recipe == "fp8_channel":
        sc = torch.empty((rows,), dtype=torch.float32, device=device)
    else:
        sc = None
    return codes, sc


class DelayedState:
    """Device-resident amax history for one tensor (delayed scaling)."""

    def __init__(self, fmt, device, hist_len=HIST_LEN, stream=None):
        self.fmt = fmt
        self.fmax = FMAX[fmt]
        n = pbs_delayed_state_bytes(hist_len)
        self.buf = torch.empty(((n + 15) // 16) * 16, dtype=torch.uint8, device=device)
        self.amax = torch.zeros(1, dtype=torch.float32, device=device)
        pbs_delayed_init(self.buf, hist_len, stream)

    @property
    def scale_inv(self):
        """The state's scale_inv word as a one-element device tensor (a view)."""
        return self.buf[4:8].view(torch.float32)

    @property
    def scale_ptr(self):
        return pbs_delayed_scale(self.buf)

    @property
    def scale_inv_ptr(self):
        return pbs_delayed_scale_inv(self.buf)

    def update(self, stream=None):
        pbs_delayed_update(self.buf, self.amax, self.fmax, stream)


class Workspace:
    """Reusable per-tensor scalars so repeated quantization allocates nothing."""

    def __init__(self, device):
        self.device = device
        self._cache = {}

    def scalars(self, key, n=3):
        t = self._cache.get(key)
        if t is None:
            t = torch.zeros(n, dtype=torch.float32, device=self.device)
            self._cache[key] = t
        return t


def _copy_scalar(dst, src, stream=None):
    """Stream-ordered device-to-device copy of one fp32 (no arithmetic)."""
    if stream is None:
        dst.copy_(src)
        return
    if isinstance(stream, int):
        stream = torch.cuda.ExternalStream(stream)
    with torch.cuda.stream(stream):
        dst.copy_(src)


def _new_scalars(dev):
    return torch.zeros(3, dtype=torch.float32, device=dev)   # amax, scale, scale_inv


def _cast_into(recipe, x, src, pass_, rmask, bufs, scal, w2d, state, stream, known_amax):
    """The amax / scale / cast calls of one recipe into the copies `bufs`
    (row codes, row scales, col codes, col scales; unused ones None).
    Returns the device tensor scale_inv the copies carry (or None)."""
    R, C = x.shape
    fmt = fmt_for(recipe, src)
    rec = RECIPES[recipe]
    row_c, row_s, col_c, col_s = bufs
    if recipe == "fp8_current":
        am = known_amax if known_amax is not None else scal[0:1]
        if known_amax is None:
            pbs_amax(x, R, C, 0, 0, am, stream)
        pbs_scale_from_amax(am, FMAX[fmt], scal[1:2], scal[2:3], stream)
        pbs_cast(rec, x, R, C, fmt, rmask, 0, 0, 0, scal[1:2], None, row_c, row_s, col_c, col_s, stream)
        return scal[2:3]
    if recipe == "fp8_delayed":
        if state is None:
            raise ValueError("delayed scaling needs a DelayedState")
        pbs_cast(rec, x, R, C, fmt, rmask, 0, 0, 0, state.scale_ptr, state.amax, row_c, row_s,
                 col_c, col_s, stream)
        # the copy keeps the scale it was cast with: a stream-ordered 4-byte
        # device copy of the state's scale_inv, which later updates replace
        _copy_scalar(scal[2:3], state.scale_inv, stream)
        return scal[2:3]
    if recipe in SUBCHANNEL + ("mxfp8", "fp8_channel", "fp8_block128_pow2"):
        pbs_cast(rec, x, R, C, fmt, rmask, int(w2d), 0, 0, None, None, row_c, row_s, col_c, col_s, stream)
        return None
    if recipe == "nvfp4":
        rht = pass_ == "wgrad"
        flags = (PBS_FLAG_RHT16 if rht else 0) | (PBS_FLAG_SR if src == "dy" else 0)
        if known_amax is not None and rht:
            raise ValueError("the Hadamard-transformed tensor's amax is not the producer's")
        am = known_amax if known_amax is not None else scal[0:1]
        if known_amax is None:
            pbs_amax(x, R, C, PBS_FLAG_RHT16 if rht else 0, RHT_SEED, am, stream)
        pbs_scale_from_amax(am, NVFP4_FMAX, scal[1:2], scal[2:3], stream)
        seed = SR_SEED if src == "dy" else RHT_SEED
        if rht and src == "dy" and RHT_SEED != SR_SEED:
            raise ValueError("one seed drives both the RHT signs and SR")
        pbs_cast(rec, x, R, C, fmt, rmask, int(w2d), flags, seed, scal[1:2], None, row_c, row_s,
                 col_c, col_s, stream)
        return scal[2:3]
    if recipe == "mxfp4":
        flags = (PBS_FLAG_RHT16 if pass_ == "wgrad" else 0) | (PBS_FLAG_SR if src == "dy" else 0)
        if flags == (PBS_FLAG_RHT16 | PBS_FLAG_SR) and RHT_SEED != SR_SEED:
            raise ValueError("one seed drives both the RHT signs and SR")
        pbs_cast(rec, x, R, C, fmt, rmask, 0, flags, SR_SEED if src == "dy" else RHT_SEED, None, None,
                 row_c, row_s, col_c, col_s, stream)
        return None
    raise ValueError(recipe)


def quantize(recipe, x, src, orient, pass_, state=None, out=None, ws=None, stream=None, known_amax=None):
    """Quantize bf16 tensor ``x`` [R, C] for use as the ``src`` operand of ``pass_``.

    Returns a QTensor whose stored shape is [R, C] (row) or [C, R] (col).
    ``out`` may be a QTensor from an earlier call with the same shape, reused
    in place.  ``state`` is a DelayedState for the delayed recipe.
    ``known_amax`` (a device fp32 of one element holding max |x|, e.g. from
    the epilogue of the GEMM that produced x) replaces the amax pass of the
    per-tensor current-scaling and NVFP4 recipes; not with the Hadamard
    transform, whose maximum is taken over the transformed values.
    """
    R, C = x.shape
    rows, cols = (R, C) if orient == "row" else (C, R)
    if recipe == "bf16":
        if orient != "row":
            raise ValueError("bf16 operands are consumed in natural storage")
        return QTensor("bf16", PBS_FMT_BF16, R, C, x)
    w2d = src in TWO_D.get(recipe, ())
    if out is None:
        codes, sc = _empty_copy(recipe, rows, cols, w2d, x.device)
        scal = _new_scalars(x.device)
        out = QTensor(recipe, fmt_for(recipe, src), rows, cols, codes, sc, scal[2:3], w2d)
        out._scal = scal
    bufs = ((out.codes, out.scales, None, None) if orient == "row" else (None, None, out.codes, out.scales))
    rmask = PBS_ROW if orient == "row" else PBS_COL
    out.tensor_scale_inv = _cast_into(recipe, x, src, pass_, rmask, bufs, out._scal, w2d, state, stream,
                                      known_amax)
    return out


def quantize_both(recipe, x, src, state=None, outs=None, stream=None, known_amax=None):
    """Row and col copies of bf16 ``x`` [R, C] from one read of x (pbs_cast
    with both orientations), for a tensor whose two copies get the same
    treatment: every recipe's weights, and the activations and gradients of
    every recipe but the 4-bit ones (whose col copies take the Hadamard
    transform, and whose gradients round stochastically).  Returns
    (row QTensor [R, C], col QTensor [C, R]); ``outs`` may be such a pair,
    reused in place."""
    if recipe == "bf16":
        raise ValueError("bf16 operands are consumed in natural storage")
    if recipe in ("nvfp4", "mxfp4") and src != "w":
        raise ValueError("the 4-bit recipes' activation and gradient copies differ (Hadamard, SR)")
    R, C = x.shape
    w2d = src in TWO_D.get(recipe, ())
    if outs is None:
        rc, rs = _empty_copy(recipe, R, C, w2d, x.device)
        cc, cs = _empty_copy(recipe, C, R, w2d, x.device)
        scal = _new_scalars(x.device)
        fmt = fmt_for(recipe, src)
        outs = (QTensor(recipe, fmt, R, C, rc, rs, scal[2:3], w2d), QTensor(recipe, fmt, C, R, cc, cs, scal[2:3], w2d))
        outs[0]._scal = outs[1]._scal = scal
    row, col = outs
    tsi = _cast_into(recipe, x, src, "fprop", PBS_ROW | PBS_COL, (row.codes, row.scales, col.codes, col.scales),
                     row._scal, w2d, state, stream, known_amax)
    row.tensor_scale_inv = col.tensor_scale_inv = tsi
    return row, col


def gemm(recipe, pass_, A, B, M, N, K, out_dtype=torch.bfloat16, C=None, stream=None, c_amax=None):
    """C[M, N] for one pass from the two operands (QTensor for quantized recipes).

    For the bf16 recipe A and B are the natural-storage bf16 tensors of the
    pass (fprop: X, W; dgrad: dY, W; wgrad: X, dY).  With ``c_amax`` (a
    device fp32 tensor of one element) the epilogue also writes max |C| there
    (pbs_gemm_amax).
    """
    dev = (A.codes if isinstance(A, QTensor) else A).device
    if C is None:
        C = torch.empty((M, N), dtype=out_dtype, device=dev)
    c_fmt = PBS_FMT_BF16 if C.dtype == torch.bfloat16 else PBS_FMT_F32
    rec = RECIPES[recipe]
    lay = LAYOUTS[pass_]
    if recipe == "bf16":
        a = A.codes if isinstance(A, QTensor) else A
        b = B.codes if isinstance(B, QTensor) else B
        args = (rec, lay, M, N, K, a, PBS_FMT_BF16, None, None, b, PBS_FMT_BF16, None, None, C, c_fmt)
    else:
        args = (rec, lay, M, N, K, A.codes, A.fmt, A.scales, A.tensor_scale_inv, B.codes, B.fmt,
                B.scales, B.tensor_scale_inv, C, c_fmt)
    if c_amax is None:
        pbs_gemm(*args, stream)
    else:
        pbs_gemm_amax(*args, c_amax, stream)
    return C


def pass_dims(pass_, M_tok, K_in, N_out):
    """(M, N, K) of the GEMM for a linear layer with X [M_tok, K_in], W [N_out, K_in]."""
    return {"fprop": (M_tok, N_out, K_in),
            "dgrad": (M_tok, K_in, N_out),
            "wgrad": (K_in, N_out, M_tok)}[pass_]


def sources(pass_, x, w, dy):
    return {"x": x, "w": w, "dy": dy}


def quantize_pass(recipe, pass_, x, w, dy, states=None, outs=None, stream=None):
    """Quantize both operands of one pass.  Returns (A, B)."""
    src = {"x": x, "w": w, "dy": dy}
    (sa, oa), (sb, ob) = ROLES[pass_]
    if recipe == "bf16":
        return src[sa], src[sb]
    states = states or {}
    outs = outs or {}
    A = quantize(recipe, src[sa], sa, oa, pass_, states.get(sa), outs.get("A"), stream=stream)
    B = quantize(recipe, src[sb], sb, ob, pass_, states.get(sb), outs.get("B"), stream=stream)
    return A, B
