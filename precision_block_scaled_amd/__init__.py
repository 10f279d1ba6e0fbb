"""Python binding of libpbs.so: block-scaled quantize-then-GEMM on MI355X.

Argument marshalling only: every function forwards to the C entry point of
the same name in ``include/pbs.h``; all arithmetic runs in the HIP kernels.
Tensors may be passed as torch tensors (their ``data_ptr()`` is used) or as
raw integer addresses; ``stream`` defaults to torch's current stream on the
current device.  A non-zero status raises ``PBSError`` with the library's
message.  If the shared library has not been built, importing this module
succeeds but the first call raises ``PBSError`` -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "PBSError", "lib", "lib_path",
    "PBS_FMT_BF16", "PBS_FMT_E4M3", "PBS_FMT_E5M2", "PBS_FMT_E2M1", "PBS_FMT_F32",
    "PBS_RECIPE_BF16", "PBS_RECIPE_FP8_CURRENT", "PBS_RECIPE_FP8_DELAYED",
    "PBS_RECIPE_FP8_BLOCK128", "PBS_RECIPE_MXFP8", "PBS_RECIPE_NVFP4", "PBS_RECIPE_MXFP4",
    "PBS_RECIPE_FP8_CHANNEL", "PBS_RECIPE_FP8_BLOCK128_1D1D", "PBS_RECIPE_FP8_BLOCK128_2D2D",
    "PBS_RECIPE_FP8_BLOCK128_POW2",
    "PBS_FPROP", "PBS_DGRAD", "PBS_WGRAD", "PBS_ROW", "PBS_COL",
    "PBS_FLAG_RHT16", "PBS_FLAG_SR",
    "pbs_amax", "pbs_scale_from_amax", "pbs_delayed_state_bytes", "pbs_delayed_init",
    "pbs_delayed_update", "pbs_delayed_scale", "pbs_delayed_scale_inv", "pbs_cast",
    "pbs_rht_cast", "pbs_gemm", "pbs_gemm_amax", "pbs_quantized_bytes", "pbs_debug_sr_encode",
    "pbs_last_error", "pbs_version",
]

PBS_OK, PBS_ERR_INVALID_ARG, PBS_ERR_SHAPE, PBS_ERR_UNSUPPORTED, PBS_ERR_HIP = range(5)
PBS_FMT_BF16, PBS_FMT_E4M3, PBS_FMT_E5M2, PBS_FMT_E2M1, PBS_FMT_F32 = range(5)
(PBS_RECIPE_BF16, PBS_RECIPE_FP8_CURRENT, PBS_RECIPE_FP8_DELAYED, PBS_RECIPE_FP8_BLOCK128,
 PBS_RECIPE_MXFP8, PBS_RECIPE_NVFP4, PBS_RECIPE_MXFP4, PBS_RECIPE_FP8_CHANNEL,
 PBS_RECIPE_FP8_BLOCK128_1D1D, PBS_RECIPE_FP8_BLOCK128_2D2D, PBS_RECIPE_FP8_BLOCK128_POW2) = range(11)
PBS_FPROP, PBS_DGRAD, PBS_WGRAD = range(3)
PBS_ROW, PBS_COL = 1, 2
PBS_FLAG_RHT16, PBS_FLAG_SR = 1, 2

lib_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpbs.so")

_c = ctypes
_vp, _i64, _i32, _u64, _f32 = _c.c_void_p, _c.c_int64, _c.c_int, _c.c_uint64, _c.c_float

# name -> (restype, argtypes); mirrors include/pbs.h
SIGNATURES = {
    "pbs_amax": (_i32, [_vp, _i64, _i64, _i32, _u64, _vp, _vp]),
    "pbs_scale_from_amax": (_i32, [_vp, _f32, _vp, _vp, _vp]),
    "pbs_delayed_state_bytes": (_i32, [_i32, _c.POINTER(_c.c_size_t)]),
    "pbs_delayed_init": (_i32, [_vp, _i32, _vp]),
    "pbs_delayed_update": (_i32, [_vp, _vp, _f32, _vp]),
    "pbs_delayed_scale": (_vp, [_vp]),
    "pbs_delayed_scale_inv": (_vp, [_vp]),
    "pbs_cast": (_i32, [_i32, _vp, _i64, _i64, _i32, _i32, _i32, _i32, _u64, _vp, _vp,
                        _vp, _vp, _vp, _vp, _vp]),
    "pbs_rht_cast": (_i32, [_i32, _vp, _i64, _i64, _u64, _i32, _u64, _vp, _vp, _vp, _vp]),
    "pbs_debug_sr_encode": (_i32, [_vp, _vp, _vp, _i64, _vp]),
    "pbs_gemm": (_i32, [_i32, _i32, _i64, _i64, _i64, _vp, _i32, _vp, _vp, _vp, _i32, _vp,
                        _vp, _vp, _i32, _vp]),
    "pbs_gemm_amax": (_i32, [_i32, _i32, _i64, _i64, _i64, _vp, _i32, _vp, _vp, _vp, _i32, _vp,
                             _vp, _vp, _i32, _vp, _vp]),
    "pbs_quantized_bytes": (_i32, [_i32, _i64, _i64, _i32, _c.POINTER(_c.c_size_t),
                                   _c.POINTER(_c.c_size_t)]),
    "pbs_last_error": (_c.c_char_p, []),
    "pbs_version": (_i32, []),
}


class PBSError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"pbs status {status}: {msg}")
        self.status = status


_lib = None


def lib():
    """The loaded libpbs.so (ctypes CDLL); raises PBSError if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise PBSError(-1, f"{lib_path} is not built; run "
                               "`python -m precision_block_scaled_amd.build` (no CPU fallback exists)")
        # torch ships its own HIP runtime under the same soname as ROCm's
        # (libamdhip64.so.7).  Loading torch first makes this library bind to
        # that one; loaded the other way round, the process would hold two
        # runtimes and the second would find no device.
        import torch  # noqa: F401
        L = _c.CDLL(lib_path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(st):
    if st != PBS_OK:
        raise PBSError(st, lib().pbs_last_error().decode())


def pbs_amax(x, rows, cols, flags, seed, amax_out, stream=None):
    _check(lib().pbs_amax(_ptr(x), rows, cols, flags, seed, _ptr(amax_out), _stream(stream)))


def pbs_scale_from_amax(amax, fmax, scale, scale_inv, stream=None):
    _check(lib().pbs_scale_from_amax(_ptr(amax), fmax, _ptr(scale), _ptr(scale_inv), _stream(stream)))


def pbs_delayed_state_bytes(hist_len):
    n = _c.c_size_t(0)
    _check(lib().pbs_delayed_state_bytes(hist_len, _c.byref(n)))
    return n.value


def pbs_delayed_init(state, hist_len, stream=None):
    _check(lib().pbs_delayed_init(_ptr(state), hist_len, _stream(stream)))


def pbs_delayed_update(state, amax, fmax, stream=None):
    _check(lib().pbs_delayed_update(_ptr(state), _ptr(amax), fmax, _stream(stream)))


def pbs_delayed_scale(state):
    return lib().pbs_delayed_scale(_ptr(state))


def pbs_delayed_scale_inv(state):
    return lib().pbs_delayed_scale_inv(_ptr(state))


def pbs_cast(recipe, x, rows, cols, fmt, orient_mask, weight_2d, flags, seed, scale, amax_out,
             row_codes, row_scales, col_codes, col_scales, stream=None):
    _check(lib().pbs_cast(recipe, _ptr(x), rows, cols, fmt, orient_mask, int(weight_2d), flags, seed,
                          _ptr(scale), _ptr(amax_out), _ptr(row_codes), _ptr(row_scales),
                          _ptr(col_codes), _ptr(col_scales), _stream(stream)))


def pbs_rht_cast(recipe, x, rows, cols, rht_seed, stochastic, sr_seed, scale, col_codes, col_scales,
                 stream=None):
    _check(lib().pbs_rht_cast(recipe, _ptr(x), rows, cols, rht_seed, int(stochastic), sr_seed, _ptr(scale),
                              _ptr(col_codes), _ptr(col_scales), _stream(stream)))


def pbs_debug_sr_encode(v, r, codes, n, stream=None):
    _check(lib().pbs_debug_sr_encode(_ptr(v), _ptr(r), _ptr(codes), n, _stream(stream)))


def pbs_gemm(recipe, layout, M, N, K, A, a_fmt, a_scale, a_tensor_scale, B, b_fmt, b_scale,
             b_tensor_scale, C, c_fmt, stream=None):
    _check(lib().pbs_gemm(recipe, layout, M, N, K, _ptr(A), a_fmt, _ptr(a_scale), _ptr(a_tensor_scale),
                          _ptr(B), b_fmt, _ptr(b_scale), _ptr(b_tensor_scale), _ptr(C), c_fmt,
                          _stream(stream)))


def pbs_gemm_amax(recipe, layout, M, N, K, A, a_fmt, a_scale, a_tensor_scale, B, b_fmt, b_scale,
                  b_tensor_scale, C, c_fmt, c_amax, stream=None):
    _check(lib().pbs_gemm_amax(recipe, layout, M, N, K, _ptr(A), a_fmt, _ptr(a_scale), _ptr(a_tensor_scale),
                               _ptr(B), b_fmt, _ptr(b_scale), _ptr(b_tensor_scale), _ptr(C), c_fmt,
                               _ptr(c_amax), _stream(stream)))


def pbs_quantized_bytes(recipe, rows, cols, weight_2d):
    a, b = _c.c_size_t(0), _c.c_size_t(0)
    _check(lib().pbs_quantized_bytes(recipe, rows, cols, int(weight_2d), _c.byref(a), _c.byref(b)))
    return a.value, b.value


def pbs_last_error():
    return lib().pbs_last_error().decode()


def pbs_version():
    return lib().pbs_version()
