"""Pins for the oracle's recipes (CPU only).

Every check ties the oracle to something other than itself: exact rational
arithmetic, closed forms, invariants that follow from the definitions,
brute force over tiny inputs, rocRAND's Philox, or the numbers the pages
print.
"""
import json
import math
import os
import shutil
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest

import workloads as W
from oracle import recipes as R
from oracle.formats import E2M1, E4M3, E5M2, bf16_to_f32, e8m0_decode
from oracle.philox import philox4x32_10, philox_word_for_index
from oracle.gemm_ref import gemm_ref, gemm_ref_bruteforce, check_gemm, ulp_bf16
from oracle.passes import pass_operands, RECIPES, ALL_RECIPES

HERE = os.path.dirname(__file__)
GOLDEN = json.load(open(os.path.join(HERE, "golden", "page_facts.json")))
FLT_MAX = float(np.finfo(np.float32).max)


# ---------------------------------------------------------------------------
# exact helpers (independent of NumPy float32 arithmetic)
# ---------------------------------------------------------------------------
def frac_to_f32(q):
    """Round an exact rational to the nearest float32 (ties to even), as a float."""
    if q == 0:
        return 0.0
    neg = q < 0
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    if Fraction(2) ** (e + 1) <= q:
        e += 1
    spacing = Fraction(2) ** (max(e, -126) - 23)
    n = q / spacing
    fl = math.floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = fl * spacing
    if val >= Fraction(2) ** 128:
        return math.inf
    out = float(val)
    return -out if neg else out


def positive_finite_bf16():
    b = np.arange(1, 0x7F80, dtype=np.uint16)
    return b, bf16_to_f32(b)


# ---------------------------------------------------------------------------
# per-tensor scale and cast
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("fmax", [448.0, 57344.0, 2688.0])
def test_scale_division_exact_over_all_bf16_amax(fmax):
    _, a = positive_finite_bf16()
    s, s_inv = R.scale_from_amax(a, fmax)
    for ai, si, sii in zip(a[::1], s, s_inv):
        want = frac_to_f32(Fraction(fmax) / Fraction(float(ai)))
        if want == math.inf:
            want = FLT_MAX
        assert float(si) == want
        assert float(sii) == frac_to_f32(1 / Fraction(want))


def test_scale_corner_cases():
    s, s_inv = R.scale_from_amax(np.float32(0.0), 448.0)
    assert s == 1.0 and s_inv == 1.0
    s, _ = R.scale_from_amax(np.float32(1e-40), 448.0)   # overflow -> FLT_MAX
    assert s == np.float32(FLT_MAX)


@pytest.mark.parametrize("s", [np.float32(1.0), np.float32(448.0 / 3.0), np.float32(2.0 ** 40 / 7)])
def test_pertensor_product_rounding_all_bf16_patterns(s):
    x = W.all_bf16_patterns().reshape(-1)
    t = bf16_to_f32(x)
    v = (t * s).astype(np.float32)
    sel = np.isfinite(v)
    for ti, vi in zip(t[sel][::7], v[sel][::7]):
        want = frac_to_f32(Fraction(float(ti)) * Fraction(float(s)))
        assert float(vi) == want or (want == 0.0 and float(vi) == 0.0)


def test_pertensor_cast_amax_element_maps_to_max_and_bounds():
    x = W.all_bf16_patterns()
    for fmt, F in (("e4m3", 448.0), ("e5m2", 57344.0)):
        codes, s_inv, a = R.quantize_current(x, fmt)
        fm = {"e4m3": E4M3, "e5m2": E5M2}[fmt]
        t = bf16_to_f32(x)
        i = np.unravel_index(np.argmax(np.abs(t)), t.shape)
        assert (codes[i] & (fm.sign_bit - 1)) == fm.max_code
        deq = fm.decode(codes) * float(s_inv)
        # relative error of a normal-range element is at most half a unit of the format
        big = np.abs(t) * (F / float(a)) >= fm.magnitudes[1 << fm.mbits]
        rel = np.abs(deq[big] - t[big]) / np.abs(t[big])
        assert rel.max() <= 2.0 ** -(fm.mbits + 1) * 1.0001


def test_pertensor_col_copy_is_transpose():
    x = W.activations(64, 96, seed=7)
    c_row, si_r, _ = R.quantize_current(x, "e4m3", "row")
    c_col, si_c, _ = R.quantize_current(x, "e4m3", "col")
    assert si_r == si_c and (c_col == c_row.T).all()


# ---------------------------------------------------------------------------
# delayed scaling
# ---------------------------------------------------------------------------
def test_delayed_closed_form_16_steps():
    base = W.activations(64, 128, seed=4)
    a0 = float(bf16_to_f32(base).__abs__().max())
    st = R.DelayedScaling("e4m3", 16)
    scales = []
    for step in range(17):
        x = W.drift(base, step)
        codes, s_inv, a = st.cast(x)
        scales.append(float(st.scale))
        # closed form of this step's amax: rounding is monotone, so the max of
        # the drifted tensor is the drifted max
        want = float(bf16_to_f32(W.f32_to_bf16_bits(np.float32(a0) * W.drift_factor(step))).reshape(-1)[0])
        assert float(a) == want
        if step < 16:
            st.update(a)
    assert scales[0] == 1.0
    hist, pos, s16, s16_inv = st.state_words()
    assert pos == 0
    amaxes = [float(bf16_to_f32(W.f32_to_bf16_bits(np.float32(a0) * W.drift_factor(k))).reshape(-1)[0])
              for k in range(16)]
    assert list(map(float, hist)) == amaxes
    # scale used at step 16 comes from the largest amax in the history: step 15's
    assert float(s16) == frac_to_f32(Fraction(448) / Fraction(amaxes[15]))
    # at step 16 the tensor grew by 1.1 over the history's max: its largest
    # element saturates, and count of saturated codes equals count of
    # elements whose exact scaled value rounds above 448
    x16 = bf16_to_f32(W.drift(base, 16)).astype(np.float64)
    codes, s_inv, _ = st.cast(W.drift(base, 16))
    n_sat = int(((codes & 0x7F) == 0x7E).sum())
    exact = np.abs(x16) * float(s16)
    assert n_sat == int((exact >= 416.0).sum())   # 416 = midpoint of 384 and 448


def test_delayed_history_wraps():
    st = R.DelayedScaling("e5m2", 4)
    for k, a in enumerate([1.0, 8.0, 2.0, 3.0, 4.0, 0.5]):
        st.update(np.float32(a))
    # window holds the last four: 2, 3, 4, 0.5
    assert sorted(map(float, st.hist)) == [0.5, 2.0, 3.0, 4.0]
    assert float(st.scale) == 57344.0 / 4.0


# ---------------------------------------------------------------------------
# sub-channel FP8
# ---------------------------------------------------------------------------
def _brute_e4m3(v):
    m = E4M3.magnitudes
    a = np.abs(v.astype(np.float64))[..., None]
    d = np.abs(a - m[None, :])
    best = d.min(axis=-1, keepdims=True)
    cand = np.where(d == best, np.arange(len(m)), 10 ** 6)
    even = np.where(cand % 2 == 0, cand, 10 ** 6).min(axis=-1)
    code = np.where(even < 10 ** 6, even, cand.min(axis=-1))
    code = np.where(a[..., 0] > 448.0, 0x7E, code)
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


@pytest.mark.parametrize("weight_2d,shape", [(False, (3, 256)), (True, (128, 256))])
def test_block128_bruteforce(weight_2d, shape):
    x = W.activations(*shape, seed=9)
    codes, s_inv = R.quantize_block128(x, "row", weight_2d)
    t = bf16_to_f32(x)
    br, bc = (128, 128) if weight_2d else (1, 128)
    for bi in range(shape[0] // br):
        for bj in range(shape[1] // bc):
            blk = t[bi * br:(bi + 1) * br, bj * bc:(bj + 1) * bc]
            a = max(abs(float(z)) for z in blk.reshape(-1))
            s = frac_to_f32(Fraction(448) / Fraction(a)) if a else 1.0
            assert float(s_inv[bi, bj]) == frac_to_f32(1 / Fraction(s))
            v = np.array([frac_to_f32(Fraction(float(z)) * Fraction(s)) for z in blk.reshape(-1)],
                         dtype=np.float32).reshape(blk.shape)
            assert (codes[bi * br:(bi + 1) * br, bj * bc:(bj + 1) * bc] == _brute_e4m3(v)).all()
            # the block maximum lands on 448
            assert (np.abs(E4M3.decode(codes[bi * br:(bi + 1) * br, bj * bc:(bj + 1) * bc])).max()
                    == 448.0)


def test_block128_outlier_stays_in_its_blocks():
    x = W.activations(4, 512, seed=2, n_outlier_channels=0)
    t = bf16_to_f32(x).copy()
    t[1, 300] = 1e4
    xo = W.f32_to_bf16_bits(t)
    c0, s0 = R.quantize_block128(x, "row")
    c1, s1 = R.quantize_block128(xo, "row")
    diff = c0 != c1
    diff_blocks = set(zip(*np.nonzero(diff)))
    assert all(r == 1 and 256 <= c < 384 for r, c in diff_blocks)
    assert (s0 != s1).sum() == 1 and s0[1, 2] != s1[1, 2]


def test_block128_2d_col_is_transpose():
    x = W.weights(256, 384, seed=5)
    cr, sr_ = R.quantize_block128(x, "row", weight_2d=True)
    cc, sc = R.quantize_block128(x, "col", weight_2d=True)
    assert (cc == cr.T).all() and (sc == sr_.T).all()


# ---------------------------------------------------------------------------
# channel-wise FP8
# ---------------------------------------------------------------------------
def test_channel_row_is_pertensor_of_each_row():
    """A row of the channel-wise copy is that row quantized on its own with
    per-tensor current scaling (pinned above exhaustively)."""
    x = W.activations(24, 384, seed=15)
    codes, s_inv = R.quantize_channel(x, "row")
    for i in range(x.shape[0]):
        c1, si1, _ = R.quantize_current(x[i:i + 1], "e4m3", "row")
        assert (codes[i] == c1[0]).all() and s_inv[i] == si1, i


def test_channel_bruteforce_and_col_copy():
    x = W.grads(3, 256, seed=16)
    codes, s_inv = R.quantize_channel(x, "row")
    t = bf16_to_f32(x)
    for i in range(3):
        a = max(abs(float(z)) for z in t[i])
        s = frac_to_f32(Fraction(448) / Fraction(a)) if a else 1.0
        assert float(s_inv[i]) == frac_to_f32(1 / Fraction(s))
        v = np.array([frac_to_f32(Fraction(float(z)) * Fraction(s)) for z in t[i]], dtype=np.float32)
        assert (codes[i] == _brute_e4m3(v)).all()
        assert np.abs(E4M3.decode(codes[i])).max() == 448.0
    cc, sc = R.quantize_channel(x, "col")
    cr, sr_ = R.quantize_channel(np.ascontiguousarray(x.T), "row")
    assert (cc == cr).all() and (sc == sr_).all()


def test_channel_outlier_stays_in_its_row_and_zero_row():
    x = W.activations(6, 256, seed=17, n_outlier_channels=0)
    t = bf16_to_f32(x).copy()
    t[2, 100] = 3e4
    t[4, :] = 0.0
    t[4, 7] = -0.0
    xo = W.f32_to_bf16_bits(t)
    c0, s0 = R.quantize_channel(x, "row")
    c1, s1 = R.quantize_channel(xo, "row")
    changed = sorted(set(np.nonzero((c0 != c1).any(axis=1))[0]) | set(np.nonzero(s0 != s1)[0]))
    assert changed == [2, 4]
    assert s1[4] == 1.0 and (c1[4] & 0x7F == 0).all() and c1[4, 7] == 0x80


# ---------------------------------------------------------------------------
# sub-channel block pairings: 1D1D and 2D2D beside the 1D2D recipe
# ---------------------------------------------------------------------------
def test_block128_pairings_choose_block_shapes_per_source():
    x = W.activations(256, 384, seed=61)
    w = W.weights(256, 384, seed=62)
    dy = W.grads(256, 256, seed=63)
    src = {"x": x, "w": w, "dy": dy}
    from oracle.passes import operand_roles
    for rec, two_d in (("fp8_block128", {"w"}), ("fp8_block128_1d1d", set()),
                       ("fp8_block128_2d2d", {"x", "w", "dy"})):
        for pass_ in ("fprop", "dgrad", "wgrad"):
            ops = pass_operands(rec, pass_, x=x, w=w, dy=dy)
            for (name, orient), q in zip(operand_roles(pass_), ops):
                c, si = R.quantize_block128(src[name], orient, weight_2d=name in two_d)
                assert q.weight_2d == (name in two_d), (rec, pass_, name)
                assert (q.codes == c).all() and (q.scale.view(np.uint32) == si.view(np.uint32)).all()
                rows, cols = q.codes.shape
                assert q.scale.shape == ((rows // 128, cols // 128) if name in two_d else (rows, cols // 128))


def test_block128_2d_scale_is_max_of_1d_scales_and_col_is_transpose():
    """A 128x128 block's stored scale fp32(1 / fp32(448 / amax)) is monotone in
    amax, so it equals the largest 1x128 stored scale of its 128 rows; a
    2D col copy is the row copy transposed, block by block."""
    x = W.grads(384, 256, seed=64)
    c1, s1 = R.quantize_block128(x, "row", weight_2d=False)
    c2, s2 = R.quantize_block128(x, "row", weight_2d=True)
    assert (s2 == s1.reshape(3, 128, 2).max(axis=1)).all()
    cc, sc = R.quantize_block128(x, "col", weight_2d=True)
    assert (cc == c2.T).all() and (sc == s2.T).all()
    # 1x128 col copy of the source: blocks along the source's rows
    cc1, sc1 = R.quantize_block128(x, "col", weight_2d=False)
    cr1, sr1 = R.quantize_block128(np.ascontiguousarray(x.T), "row", weight_2d=False)
    assert (cc1 == cr1).all() and (sc1 == sr1).all()


# ---------------------------------------------------------------------------
# sub-channel FP8 with power-of-two block scales
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("weight_2d,shape", [(False, (3, 256)), (True, (128, 256))])
def test_block128_pow2_bruteforce(weight_2d, shape):
    """Per block: the E8M0 code is the smallest of all 255 finite codes whose
    power of two brings every element within 448 (exact rationals), and each
    code is the brute-force nearest-even E4M3 code of the exactly scaled value."""
    x = W.activations(*shape, seed=19)
    t = bf16_to_f32(x)
    t[0, :128] *= np.float32(2.0 ** -100)         # a block that needs a large scale
    x = W.f32_to_bf16_bits(t)
    t = bf16_to_f32(x)
    codes, e8 = R.quantize_block128_pow2(x, "row", weight_2d)
    br, bc = (128, 128) if weight_2d else (1, 128)
    assert e8.shape == (shape[0] // br, shape[1] // bc) and e8.dtype == np.uint8
    for bi in range(shape[0] // br):
        for bj in range(shape[1] // bc):
            blk = t[bi * br:(bi + 1) * br, bj * bc:(bj + 1) * bc].reshape(-1)
            a = max(abs(Fraction(float(z))) for z in blk)
            c = next(c for c in range(255) if a <= 448 * Fraction(2) ** (c - 127))
            assert int(e8[bi, bj]) == c
            sc = Fraction(2) ** (127 - c)
            v = np.array([frac_to_f32(Fraction(float(z)) * sc) for z in blk], dtype=np.float32)
            got = codes[bi * br:(bi + 1) * br, bj * bc:(bj + 1) * bc].reshape(-1)
            assert (got == _brute_e4m3(v)).all()
            # the scaled block maximum lies in (224, 448]: half the scale would saturate
            m = np.abs(E4M3.decode(got)).max()
            assert 224.0 <= m <= 448.0 and (c == 0 or a * sc > 224)


def test_block128_pow2_scale_is_power_of_two_below_fp32_scale():
    """2**-e is the largest power of two not above the exact 448 / amax_b
    (the fp32 sub-channel scale before rounding)."""
    x = W.grads(8, 1024, seed=20)
    codes, e8 = R.quantize_block128_pow2(x, "row")
    a_b = np.abs(bf16_to_f32(x)).reshape(8, 8, 128).max(axis=-1)
    for a, c in zip(a_b.reshape(-1), e8.reshape(-1)):
        q = Fraction(448) / Fraction(float(a))
        s = Fraction(2) ** (127 - int(c))
        assert s <= q < 2 * s


def test_block128_pow2_reduces_to_mxfp8_when_sub_blocks_share_the_max():
    """When every 32-value sub-block holds its 128-block's maximum magnitude,
    the MXFP8 rule gives each sub-block the 128-block's exponent: codes agree
    with the MXFP8 oracle and its four scales repeat the block's one."""
    t = bf16_to_f32(W.activations(16, 512, seed=21)).copy()
    blocks = t.reshape(16, 4, 4, 32)
    bmax = np.abs(blocks).max(axis=(2, 3))
    blocks[:, :, :, 0] = -bmax[:, :, None]       # same magnitude in every sub-block
    x = W.f32_to_bf16_bits(blocks.reshape(16, 512))
    cp, ep = R.quantize_block128_pow2(x, "row")
    cm, em = R.quantize_mxfp8(x, "row")
    assert (cp == cm).all() and (np.repeat(ep, 4, axis=1) == em).all()
    # without that structure the sub-blocks may take smaller exponents
    x2 = W.activations(16, 512, seed=22)
    ep2 = R.quantize_block128_pow2(x2, "row")[1]
    em2 = R.quantize_mxfp8(x2, "row")[1]
    assert (np.repeat(ep2, 4, axis=1) >= em2).all() and (np.repeat(ep2, 4, axis=1) > em2).any()


def test_block128_pow2_2d_is_max_of_1d_and_col_is_transpose():
    x = W.weights(384, 256, seed=23)
    c1, e1 = R.quantize_block128_pow2(x, "row", weight_2d=False)
    c2, e2 = R.quantize_block128_pow2(x, "row", weight_2d=True)
    assert (e2 == e1.reshape(3, 128, 2).max(axis=1)).all()
    cc, ec = R.quantize_block128_pow2(x, "col", weight_2d=True)
    assert (cc == c2.T).all() and (ec == e2.T).all()
    cc1, ec1 = R.quantize_block128_pow2(x, "col", weight_2d=False)
    cr1, er1 = R.quantize_block128_pow2(np.ascontiguousarray(x.T), "row", weight_2d=False)
    assert (cc1 == cr1).all() and (ec1 == er1).all()
    # dequantization: code value times 2**e exactly, per 128x128 block
    d = R.dequant_block128_pow2(c2, e2, weight_2d=True)
    assert d[0, 0] == float(E4M3.decode(c2[:1, :1])[0, 0]) * 2.0 ** (int(e2[0, 0]) - 127)


def test_block128_pow2_pairing_and_zero_block():
    x = W.activations(256, 384, seed=24)
    w = W.weights(256, 384, seed=25)
    dy = W.grads(256, 256, seed=26)
    from oracle.passes import operand_roles
    src = {"x": x, "w": w, "dy": dy}
    for pass_ in ("fprop", "dgrad", "wgrad"):
        ops = pass_operands("fp8_block128_pow2", pass_, x=x, w=w, dy=dy)
        for (name, orient), q in zip(operand_roles(pass_), ops):
            c, e = R.quantize_block128_pow2(src[name], orient, weight_2d=name == "w")
            assert q.weight_2d == (name == "w") and (q.codes == c).all() and (q.scale == e).all()
    z = np.zeros((2, 256), np.uint16)
    z[1, 5] = 0x8000                               # -0
    c, e = R.quantize_block128_pow2(z, "row")
    assert (e == 0).all() and (c & 0x7F == 0).all() and c[1, 5] == 0x80


# ---------------------------------------------------------------------------
# MXFP8
# ---------------------------------------------------------------------------
def test_mx_exponent_closed_form_all_bf16():
    _, a = positive_finite_bf16()
    got = R.mx_block_exponent_code(a).astype(np.int64) - 127
    f, ex = np.frexp(a.astype(np.float64))          # a = f * 2**ex, f in [0.5, 1)
    mant = 2 * f                                     # in [1, 2)
    E = ex - 1
    want = np.clip(E - 8 + (mant > 1.75), -127, 127)
    assert (got == want).all()
    assert R.mx_block_exponent_code(np.float32(0.0)) == 0


def test_mx_no_saturation_and_half_scale_would():
    x = W.activations(16, 512, seed=12)
    codes, e8 = R.quantize_mxfp8(x)
    t = bf16_to_f32(x).astype(np.float64).reshape(16, 16, 32)
    scale = e8m0_decode(e8)[..., None]
    assert (np.abs(t) / scale <= 448.0).all()
    bm = np.abs(t).max(axis=-1)
    e = e8.astype(np.int64) - 127
    assert ((bm / np.ldexp(1.0, e - 1) > 448.0) | (e == -127)).all()
    deq = R.dequant_mxfp8(codes, e8).reshape(16, 16, 32)
    assert np.all(np.abs(deq - t) <= scale * 2.0 ** -4 * np.maximum(np.abs(t) / scale, 2.0 ** -6) + 1e-300)


# ---------------------------------------------------------------------------
# NVFP4
# ---------------------------------------------------------------------------
def test_nvfp4_block_scale_bruteforce_and_global_block():
    x = W.activations(32, 256, seed=13)
    t = bf16_to_f32(x)
    A = R.amax(t)
    S_enc, S_dec = R.nvfp4_tensor_scales(A)
    assert float(S_enc) == frac_to_f32(Fraction(2688) / Fraction(float(A)))
    packed, d = R.quantize_nvfp4(t, S_enc)
    a_b = np.abs(t).reshape(32, 16, 16).max(axis=-1)
    for i in range(32):
        for j in range(16):
            q = frac_to_f32(Fraction(frac_to_f32(Fraction(float(a_b[i, j])) / 6)) * Fraction(float(S_enc)))
            assert d[i, j] == _brute_e4m3(np.array([q], dtype=np.float32))[0]
    # the block holding the tensor amax gets the largest E4M3 scale
    i, j = np.unravel_index(np.argmax(a_b), a_b.shape)
    assert d[i, j] == 0x7E


def test_nvfp4_storage_matches_page_accounting():
    n_facts = GOLDEN["nvfp4"]
    for rows, cols in ((16, 4096), (64, 16384)):
        x = W.activations(rows, cols, seed=1)
        t = bf16_to_f32(x)
        packed, d = R.quantize_nvfp4(t, R.nvfp4_tensor_scales(R.amax(t))[0])
        n = rows * cols
        nbytes = packed.nbytes + d.nbytes + 4
        assert nbytes == n // 2 + n // 16 + 4
        bits = 8 * nbytes / n
        assert abs(bits - (4.5 + 32 / n)) < 1e-12
        assert round(bits, 2) == n_facts["approx_bits_per_value"]
    assert round(16 / 4.5, 1) in (3.5, 3.6) and abs(16 / 4.5 - n_facts["approx_memory_reduction_vs_fp16"]) < 0.1
    assert round(8 / 4.5, 1) == n_facts["approx_memory_reduction_vs_fp8"]


def test_nvfp4_dequant_error_within_half_unit():
    x = W.activations(16, 512, seed=21)
    t = bf16_to_f32(x)
    S_enc, S_dec = R.nvfp4_tensor_scales(R.amax(t))
    packed, d = R.quantize_nvfp4(t, S_enc)
    deq = R.dequant_nvfp4(packed, d, S_dec)
    # each element is within half an E2M1 step (at most 1 unit for the 4..6
    # gap) of its scaled value, up to the fp32 roundings of the scales
    dd = np.repeat(E4M3.decode(d), 16, axis=1) * float(S_dec)
    err = np.abs(deq - t) / np.where(dd > 0, dd, 1)
    assert err.max() <= 1.0 + 1e-5


def test_nvfp4_zero_block_and_sign():
    t = np.zeros((2, 32), dtype=np.float32)
    t[0, :16] = -0.0
    t[1, 16:] = 5.0
    packed, d = R.quantize_nvfp4(t, R.nvfp4_tensor_scales(R.amax(t))[0])
    codes = R.unpack_e2m1(packed)
    assert (d[0] == 0).all() and (codes[0, :16] == 8).all() and (codes[0, 16:] == 0).all()
    assert d[1, 1] == 0x7E and (codes[1, 16:] == 7).all()


def test_nvfp4_2d_col_is_transpose():
    x = W.weights(64, 96, seed=8)
    t = bf16_to_f32(x)
    S_enc = R.nvfp4_tensor_scales(R.amax(t))[0]
    pr, dr = R.quantize_nvfp4(t, S_enc, weight_2d=True)
    pc, dc = R.quantize_nvfp4(np.ascontiguousarray(t.T), S_enc, weight_2d=True)
    assert (R.unpack_e2m1(pc) == R.unpack_e2m1(pr).T).all() and (dc == dr.T).all()


# ---------------------------------------------------------------------------
# MXFP4 (E2M1 values, E8M0 scale per 32)
# ---------------------------------------------------------------------------
def test_mx4_exponent_closed_form_all_bf16():
    _, a = positive_finite_bf16()
    got = R.mx4_block_exponent_code(a).astype(np.int64) - 127
    f, ex = np.frexp(a.astype(np.float64))          # a = f * 2**ex, f in [0.5, 1)
    mant = 2 * f                                     # in [1, 2)
    E = ex - 1
    # 6 * 2**e >= mant * 2**E  <=>  e >= E - 2 + log2(mant / 1.5)
    want = np.clip(E - 2 + (mant > 1.5), -127, 127)
    assert (got == want).all()
    assert R.mx4_block_exponent_code(np.float32(0.0)) == 0


def _brute_e2m1_code(q):
    """Nearest E2M1 magnitude to |q| (an exact Fraction), ties to the even code; sign bit 8."""
    mags = [Fraction(float(m)) for m in E2M1.magnitudes]
    a = abs(q)
    if a > 6:
        code = 7
    else:
        d = [abs(a - m) for m in mags]
        best = min(d)
        cands = [i for i, di in enumerate(d) if di == best]
        code = min(cands, key=lambda i: (i % 2, i))
    return code | (8 if q < 0 else 0)


def _mx4_brute_block(vals):
    """(E8M0 code, E2M1 codes) of one 32-value block by direct search, exact arithmetic."""
    fr = [Fraction(float(v)) for v in vals]
    a = max(abs(f) for f in fr)
    e = next(e for e in range(-127, 128) if a <= 6 * Fraction(2) ** e)
    codes = []
    for v, f in zip(vals, fr):
        if f == 0:
            codes.append(8 if np.signbit(v) else 0)
        else:
            codes.append(_brute_e2m1_code(Fraction(frac_to_f32(f / Fraction(2) ** e))))
    return e + 127, codes


def test_mxfp4_bruteforce():
    rng = np.random.default_rng(31)
    t = bf16_to_f32(W.activations(6, 128, seed=31)).copy()
    t[0, :32] = 0.0
    t[0, 5] = -0.0
    t[1, :32] = rng.choice(np.float32([0.5, 1.5, 3, 6]), 32) * np.float32(2.0 ** 10)  # max 6*2^10: e = 10
    t[1, 3] = 6 * 2.0 ** 10
    t[1, 32:64] *= 0
    t[1, 40] = np.float32(6 * 2.0 ** 10) * np.float32(1 + 2 ** -7)              # just above: e = 11
    t[2, 64:96] = np.float32(2.0 ** -133)                                        # bf16 subnormals: e = -127
    t[2, 70] = np.float32(2.0 ** -126)
    t[3, 96:128] = np.float32(1.25) * rng.choice([-1, 1], 32)                    # ties at 1.25 -> 1.0
    t[4, :32] = np.float32(3e38) * rng.random(32, dtype=np.float32)
    packed, e8 = R.quantize_mxfp4(t)
    codes = R.unpack_e2m1(packed)
    assert codes.shape == t.shape and e8.shape == (6, 4)
    for i in range(t.shape[0]):
        for b in range(4):
            ce, cc = _mx4_brute_block(t[i, 32 * b:32 * b + 32])
            assert e8[i, b] == ce, (i, b)
            assert list(codes[i, 32 * b:32 * b + 32]) == cc, (i, b)
    assert e8[1, 0] == 127 + 10 and e8[1, 1] == 127 + 11 and e8[2, 2] == 0


def test_mxfp4_no_saturation_and_half_scale_would():
    x = W.activations(16, 512, seed=22)
    t = bf16_to_f32(x)
    packed, e8 = R.quantize_mxfp4(t)
    tt = t.astype(np.float64).reshape(16, 16, 32)
    scale = e8m0_decode(e8)[..., None]
    assert (np.abs(tt) / scale <= 6.0).all()
    bm = np.abs(tt).max(axis=-1)
    e = e8.astype(np.int64) - 127
    assert ((bm / np.ldexp(1.0, e - 1) > 6.0) | (e == -127)).all()
    deq = R.dequant_mxfp4(packed, e8).reshape(16, 16, 32)
    # within half an E2M1 step of the scaled value: 0.25 below 2, |v|/4 above
    v = np.abs(tt) / scale
    assert np.all(np.abs(deq - tt) <= scale * np.maximum(0.25, v / 4))


def test_mxfp4_sr_extremes_and_grid():
    t = bf16_to_f32(W.grads(4, 64, seed=23))
    _, e8 = R.quantize_mxfp4(t)
    scale = e8m0_decode(e8)
    zeros = np.zeros(t.shape, np.uint32)
    ones = np.full(t.shape, 0xFFFFFFFF, np.uint32)
    up = E2M1.decode(R.unpack_e2m1(R.quantize_mxfp4(t, sr_random=zeros)[0]))
    dn = E2M1.decode(R.unpack_e2m1(R.quantize_mxfp4(t, sr_random=ones)[0]))
    mags = E2M1.magnitudes
    for i in range(t.shape[0]):
        for j in range(t.shape[1]):
            v = Fraction(float(t[i, j])) / Fraction(float(scale[i, j // 32]))
            a = abs(v)
            lo = max(float(m) for m in mags if Fraction(float(m)) <= a)
            hi = min([float(m) for m in mags if Fraction(float(m)) >= a])
            sgn = -1.0 if v < 0 else 1.0
            assert up[i, j] == sgn * hi and dn[i, j] == sgn * lo, (i, j, float(v))
    # on-grid blocks never move
    g = np.tile(np.float32([0, 0.5, 1, 1.5, 2, 3, 4, 6]), 4)[None, :] * np.float32(0.25)
    r = philox_word_for_index(np.arange(32), 42)[None, :]
    p, e = R.quantize_mxfp4(g, sr_random=r)
    assert (R.dequant_mxfp4(p, e) == g).all()


@pytest.mark.parametrize("rec", ["nvfp4", "mxfp4"])
def test_fp4_wgrad_with_rht_tracks_exact_product(rec):
    """Both Wgrad operands carry the same orthogonal transform, so their product
    still approximates X^T dY (a transform on one side only would not)."""
    x = W.activations(256, 128, seed=25)
    dy = W.grads(256, 96, seed=26)
    A, B = pass_operands(rec, "wgrad", x=x, w=None, dy=dy)
    assert A.extra["rht"] and B.extra["rht"] and B.extra["sr"] and not A.extra["sr"]
    ref = bf16_to_f32(x).astype(np.float64).T @ bf16_to_f32(dy).astype(np.float64)
    c, _ = gemm_ref(A.dequant(), B.dequant())
    rel = np.linalg.norm(c - ref) / np.linalg.norm(ref)
    # typical over SR draws: NVFP4 0.17, MXFP4 0.19-0.20 (power-of-two 32-blocks)
    assert rel < (0.2 if rec == "nvfp4" else 0.25), rel
    A0 = pass_operands(rec, "fprop", x=np.ascontiguousarray(x.T), w=np.ascontiguousarray(dy.T),
                       dy=None)[0]
    c0, _ = gemm_ref(A0.dequant(), B.dequant())
    assert np.linalg.norm(c0 - ref) / np.linalg.norm(ref) > 0.5


def test_mxfp4_coarser_than_nvfp4():
    """NVFP4's 16-value blocks with fractional scales lose less than MXFP4's 32-value
    power-of-two blocks on the same activations (the reason the pages give for NVFP4)."""
    t = bf16_to_f32(W.activations(64, 1024, seed=24))
    S_enc, S_dec = R.nvfp4_tensor_scales(R.amax(t))
    e_nv = np.abs(R.dequant_nvfp4(*R.quantize_nvfp4(t, S_enc), S_dec) - t).mean()
    e_mx = np.abs(R.dequant_mxfp4(*R.quantize_mxfp4(t)) - t).mean()
    assert e_nv < e_mx


# ---------------------------------------------------------------------------
# Philox and stochastic rounding
# ---------------------------------------------------------------------------
def _rocrand_helper():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND cross-check")
    d = tempfile.mkdtemp(prefix="pbs_philox_")
    exe = os.path.join(d, "philox_rocrand")
    subprocess.run([hipcc, "-O1", os.path.join(HERE, "helpers", "philox_rocrand.cpp"), "-o", exe],
                   check=True, capture_output=True)
    return exe


def test_philox_matches_rocrand():
    exe = _rocrand_helper()
    rng = np.random.default_rng(77)
    cases = [(42, 0, i, 0, 0, 0) for i in range(64)]
    cases += [(42, 0, j, 0, 1, 0) for j in range(16)]
    cases += [(42, 0, 5, 3, 0, 0), (42, 0, 0xFFFFFFFF, 1, 0, 0)]
    for _ in range(64):
        k0, k1, c0, c2, c3 = (int(v) for v in rng.integers(0, 2 ** 32, 5))
        cases.append((k0, k1, c0, int(rng.integers(0, 2 ** 28)), c2, c3))
    inp = "\n".join(" ".join(str(v) for v in c) for c in cases) + "\n"
    out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout.split("\n")
    for c, line in zip(cases, out):
        k0, k1, c0, c1, c2, c3 = c
        ours = philox4x32_10(c0, c1, c2, c3, k0, k1)
        assert " ".join("%08x" % int(w) for w in ours) == line.strip(), c


def test_sr_word_statistics():
    r = philox_word_for_index(np.arange(1 << 20), 42)
    # 16-bin chi-square on the top 4 bits; 15 dof, p = 1e-6 cut ~ 55
    counts = np.bincount((r >> 28).astype(np.int64), minlength=16)
    exp = len(r) / 16
    chi2 = ((counts - exp) ** 2 / exp).sum()
    assert chi2 < 55
    bits = np.unpackbits(r.view(np.uint8)).reshape(-1, 32).mean(axis=0)
    assert np.all(np.abs(bits - 0.5) < 5 * 0.5 / math.sqrt(len(r)))
    # the four words of one call are not correlated with each other
    w = r.reshape(-1, 4).astype(np.float64) / 2 ** 32 - 0.5
    c = np.corrcoef(w.T)
    assert np.all(np.abs(c[np.triu_indices(4, 1)]) < 5 / math.sqrt(w.shape[0]))


def test_sr_word_is_a_word_of_the_call_for_index_over_4():
    """Element i takes word i % 4 of the call with counter i // 4 (the
    generator itself is checked against rocRAND above)."""
    for i in (0, 1, 2, 3, 4, 7, 1001, (1 << 32) * 4 + 6, (5 << 34) + 3):
        q, k = i // 4, i % 4
        want = philox4x32_10(q & 0xFFFFFFFF, q >> 32, 0, 0, 42, 0)[k]
        assert philox_word_for_index(i, 42) == want, i
    # seeds above 32 bits reach the second key word
    assert philox_word_for_index(9, 1 << 40) == philox4x32_10(2, 0, 0, 0, 0, 1 << 8)[1]


def test_sr_threshold_exact():
    vals = np.array([0.1, 0.3, 0.7, 1.2, 1.6, 2.2, 2.9, 3.3, 4.4, 5.9, 1e-30, 4.000001],
                    dtype=np.float32)
    mags = [Fraction(float(m)) for m in E2M1.magnitudes]
    for v in vals:
        a = Fraction(float(v))
        lo = max(m for m in mags if m <= a)
        hi = min(m for m in mags if m > a)
        T = math.ceil((a - lo) / (hi - lo) * 2 ** 32)
        lo_code = int(E2M1.encode(np.float32(float(lo)))[()])
        hi_code = int(E2M1.encode(np.float32(float(hi)))[()])
        if T >= 1:
            assert R.sr_e2m1(np.array([v]), np.array([T - 1], dtype=np.uint32))[0] == hi_code
        if T <= 2 ** 32 - 1:
            assert R.sr_e2m1(np.array([v]), np.array([T], dtype=np.uint32))[0] == lo_code
        # sign symmetry
        assert R.sr_e2m1(np.array([-v]), np.array([0], dtype=np.uint32))[0] == (hi_code | 8)


def test_sr_grid_fixed_and_unbiased():
    grid = E2M1.magnitudes.astype(np.float32)
    r = philox_word_for_index(np.arange(4096), 42)
    for g in grid:
        assert (E2M1.decode(R.sr_e2m1(np.full(4096, g, dtype=np.float32), r)) == g).all()
    assert (R.sr_e2m1(np.full(8, 7.5, np.float32), r[:8]) == 7).all()
    n = 1 << 20
    r = philox_word_for_index(np.arange(n), 42)
    for v in (0.3, 1.3, 2.6, 4.9):
        out = E2M1.decode(R.sr_e2m1(np.full(n, v, dtype=np.float32), r))
        mags = E2M1.magnitudes
        lo = mags[mags <= v].max()
        hi = mags[mags > v].min()
        p = (np.float32(v) - lo) / (hi - lo)
        sigma = (hi - lo) * math.sqrt(p * (1 - p) / n)
        assert abs(out.mean() - float(np.float32(v))) < 4 * sigma


def test_sr_counter_is_logical_index_in_both_copies():
    r_row = R.sr_random_for((32, 48), "row")
    r_col = R.sr_random_for((32, 48), "col")
    assert (r_col == r_row.T).all()
    i = 3 * 48 + 5
    assert r_row[3, 5] == philox4x32_10(i // 4, 0, 0, 0, 42, 0)[i % 4]


# ---------------------------------------------------------------------------
# RHT16
# ---------------------------------------------------------------------------
def test_rht_matches_hadamard_popcount_formula():
    eye = np.eye(16, dtype=np.float32)
    y = R.rht16_along_rows(eye)                 # column j = 1/4 H D e_j
    sig = R.rht_signs(42)
    for i in range(16):
        for j in range(16):
            h = (-1) ** bin(i & j).count("1")
            assert y[i, j] == np.float32(0.25 * h * sig[j])
    # signs: bit 0 of word 0 of Philox(key (42,0), counter (j, 0, 1, 0))
    w = philox4x32_10(np.arange(16), 0, 1, 0, 42, 0)[0]
    assert (sig == np.where(w & 1, -1.0, 1.0)).all()
    assert set(np.unique(sig)) <= {-1.0, 1.0}
    # orthogonal: T T^T = I exactly
    assert (y.astype(np.float64) @ y.T.astype(np.float64) == np.eye(16)).all()


def test_rht_preserves_wgrad_product():
    x = bf16_to_f32(W.activations(256, 8, seed=3)).astype(np.float32)
    dy = bf16_to_f32(W.grads(256, 6, seed=4)).astype(np.float32)
    tx = R.rht16_along_rows(x).astype(np.float64)
    td = R.rht16_along_rows(dy).astype(np.float64)
    ref = x.astype(np.float64).T @ dy.astype(np.float64)
    got = tx.T @ td
    bound = np.abs(x.astype(np.float64)).T @ np.abs(dy.astype(np.float64))
    assert np.all(np.abs(got - ref) <= 1e-6 * bound + 1e-30)


def test_rht_inverse():
    x = bf16_to_f32(W.activations(32, 4, seed=6))
    y = R.rht16_along_rows(x).astype(np.float64)
    H = np.array([[(-1) ** bin(i & j).count("1") for j in range(16)] for i in range(16)], float)
    D = np.diag(R.rht_signs(42).astype(np.float64))
    back = np.concatenate([D @ H @ y[g * 16:(g + 1) * 16] / 4 for g in range(2)])
    assert np.allclose(back, x, rtol=1e-6, atol=0)


# ---------------------------------------------------------------------------
# GEMM reference
# ---------------------------------------------------------------------------
def test_gemm_ref_bruteforce_and_special_cases():
    rng = np.random.default_rng(0)
    a = rng.standard_normal((7, 33))
    b = rng.standard_normal((5, 33))
    c, bnd = gemm_ref(a, b)
    assert np.allclose(c, gemm_ref_bruteforce(a, b), rtol=1e-13, atol=1e-13)
    assert (bnd >= np.abs(c)).all()
    perm = np.eye(33)[rng.permutation(33)]
    c2, _ = gemm_ref(a, perm)          # B = permutation: exact copy of permuted A
    assert (c2 == a @ perm.T).all() and (np.sort(c2, axis=1) == np.sort(a, axis=1)).all()
    ok, tol, err = check_gemm(c * (1 + 5e-6), c, bnd, False)
    assert ok.all()
    ok, _, _ = check_gemm(c + 2e-5 * bnd, c, bnd, False)
    assert not ok.any()


def test_ulp_bf16():
    assert ulp_bf16(1.0) == 2.0 ** -7
    assert ulp_bf16(1.99) == 2.0 ** -7
    assert ulp_bf16(2.0) == 2.0 ** -6
    assert ulp_bf16(-3.0) == 2.0 ** -6
    assert ulp_bf16(0.0) == 2.0 ** -133


def test_tiny_case_all_recipes_gemm_close_to_bf16_product():
    a, w = W.tiny_current_case(0)
    x = a                         # [256, 512]
    dy = W.grads(256, 256, seed=3)
    exact = {p: None for p in ("fprop",)}
    ta = bf16_to_f32(a).astype(np.float64)
    tw = bf16_to_f32(w).astype(np.float64)
    ref = ta @ tw.T
    errs = {}
    for rec in ALL_RECIPES:
        st = None
        if rec == "fp8_delayed":
            st = {"x": R.DelayedScaling("e4m3"), "w": R.DelayedScaling("e4m3")}
            st["x"].update(R.amax(x))
            st["w"].update(R.amax(w))
        A, B = pass_operands(rec, "fprop", x=x, w=w, dy=dy, delayed_states=st)
        c, _ = gemm_ref(A.dequant(), B.dequant())
        errs[rec] = np.abs(c - ref).max() / np.abs(ref).max()
    assert errs["bf16"] == 0.0
    # finer granularity tracks the bf16 product more closely
    assert errs["fp8_block128"] <= errs["fp8_current"] * 1.05
    assert errs["mxfp8"] < 0.1 and errs["nvfp4"] < 0.3 and errs["mxfp4"] < 0.3
    # 1x128 weight blocks track at least as well as 128x128 ones, which track
    # at least as well as 128x128 blocks on the activations too
    assert errs["fp8_block128_1d1d"] <= errs["fp8_block128"] * 1.05
    assert errs["fp8_block128"] <= errs["fp8_block128_2d2d"] * 1.05
    # power-of-two block scales use at most one binade less of E4M3's range
    assert errs["fp8_block128_pow2"] < 0.1
    # one scale per row tracks at least as well as one per tensor
    assert errs["fp8_channel"] <= errs["fp8_current"] * 1.05 and errs["fp8_channel"] < 0.1
    for rec in ("fp8_current", "fp8_delayed", "fp8_block128", "mxfp8"):
        assert errs[rec] < 0.1, (rec, errs[rec])


# ---------------------------------------------------------------------------
# shapes and inputs
# ---------------------------------------------------------------------------
def test_codonfm_shapes_match_page():
    g = GOLDEN["codonfm_5b"]
    c = W.CODONFM_5B
    assert c["micro_batch"] * c["seq_len"] == g["tokens_M"] == 15872
    shapes = W.codonfm_shapes()
    assert len(shapes) == g["n_gemm_shapes"] == 12
    assert len({(s.layer, s.pass_) for s in shapes}) == 12
    d = {(s.layer, s.pass_): (s.m, s.k, s.n) for s in shapes}
    assert d[("qkv", "fprop")] == (15872, 4096, 12288)
    assert d[("qkv", "dgrad")] == (15872, 12288, 4096)     # K and N swapped
    assert d[("attn_out", "fprop")] == (15872, 4096, 4096)
    assert d[("mlp_up", "fprop")] == (15872, 4096, 16384)
    assert d[("mlp_down", "fprop")] == (15872, 16384, 4096)
    assert d[("mlp_down", "wgrad")] == (16384, 15872, 4096)
    total = sum(s.flop for s in shapes)
    assert abs(total / 1e12 - 19.173) < 1e-3
    assert len(W.codonfm_shapes(tokens=32 * 1024)) == 12
    ll = W.gemm_shapes(**{k: v for k, v in W.LLAMA3_8B_LAYER.items()})
    dl = {(s.layer, s.pass_): (s.m, s.k, s.n) for s in ll}
    assert dl[("qkv", "fprop")] == (8192, 4096, 6144)
    assert dl[("mlp_up", "fprop")] == (8192, 4096, 28672)
    assert dl[("mlp_down", "fprop")] == (8192, 14336, 4096)


def test_inputs_deterministic_and_rne():
    import torch
    a1 = W.activations(600, 64, seed=1)
    a2 = W.activations(600, 64, seed=1)
    assert (a1 == a2).all()
    assert not (W.activations(600, 64, seed=2) == a1).all()
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 77
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (W.f32_to_bf16_bits(x) == ref).all()
    t = bf16_to_f32(W.activations(512, 1024, seed=1))
    big = np.abs(t).max(axis=0) > 50
    assert big.sum() == 8
    g = bf16_to_f32(W.grads(256, 256))
    assert abs(np.median(np.abs(g)) - 0.765e-3) < 0.1e-3     # median |t_3| = 0.765


# ---------------------------------------------------------------------------
# NVFP4: exact worked examples and element-wise brute force
# ---------------------------------------------------------------------------
def _frac_nearest_e2m1(v):
    a = abs(Fraction(float(v)))
    mags = [Fraction(float(m)) for m in E2M1.magnitudes]
    if a > 6:
        c = 7
    else:
        best = min(range(8), key=lambda i: (abs(a - mags[i]), i % 2))
        c = best
    return c | (8 if np.signbit(v) else 0)


def test_nvfp4_ties_worked_example():
    # global amax 21 -> S_enc = 2688 / 21 = 128 exactly; a block whose max is 6
    # gets d = E4M3(6 / 6 * 128) = 128 and e_b = 128 / 128 = 1, so every
    # element is encoded as itself: E2M1 midpoints must go to the even code.
    blk = np.array([6.0, 2.5, 0.25, 0.75, 1.25, 1.75, 3.5, 5.0,
                    -2.5, -0.25, -5.0, 0.0, 21.0 / 64, 4.0, 1.0, -6.0], dtype=np.float32)
    t = np.stack([blk, np.r_[np.full(15, 1.0), 21.0].astype(np.float32)])
    S_enc, S_dec = R.nvfp4_tensor_scales(R.amax(t))
    assert S_enc == 128.0
    packed, d = R.quantize_nvfp4(t, S_enc)
    assert d[0, 0] == E4M3.encode(np.float32(128.0))
    codes = R.unpack_e2m1(packed)[0]
    want = [6.0, 2.0, 0.0, 1.0, 1.0, 2.0, 4.0, 4.0, -2.0, -0.0, -4.0, 0.0, 0.5, 4.0, 1.0, -6.0]
    got = E2M1.decode(codes)
    assert list(got) == want
    assert np.signbit(got[9])


def test_nvfp4_block_scale_rounding_order():
    # d = enc_E4M3(fp32(fp32(a_b / 6) * S_enc)): the division by 6 rounds
    # first.  Search pairs (a_b, S) where doing the product first would give
    # another E4M3 code, and check the oracle follows the stated order.
    mids = (E4M3.magnitudes[:-1] + E4M3.magnitudes[1:]) / 2
    found = []
    bf = bf16_to_f32(np.arange(0x3F80, 0x4000, dtype=np.uint16))       # a_b in [1, 2)
    for M in mids[(mids > 1) & (mids < 400)][::3]:
        for a in bf:
            S = np.float32(6 * M / float(a))
            stated = frac_to_f32(Fraction(frac_to_f32(Fraction(float(a)) / 6)) * Fraction(float(S)))
            other = frac_to_f32(Fraction(frac_to_f32(Fraction(float(a)) * Fraction(float(S)))) / 6)
            cs = _brute_e4m3(np.array([stated], np.float32))[0]
            co = _brute_e4m3(np.array([other], np.float32))[0]
            if cs != co:
                found.append((a, S, cs))
        if len(found) >= 12:
            break
    assert len(found) >= 4
    for a, S, cs in found:
        t = np.zeros((1, 16), np.float32)
        t[0, 3] = a
        _, d = R.quantize_nvfp4(t, S)
        assert d[0, 0] == cs


@pytest.mark.parametrize("seed", [0, 1])
def test_nvfp4_elements_bruteforce(seed):
    # bf16 magnitudes 2**-21 .. 16 in shuffled 16-blocks, both signs
    b = np.arange(0x3500, 0x4180, dtype=np.uint16)
    b = np.concatenate([b, b | 0x8000])
    rng = np.random.default_rng(seed)
    b = b[rng.permutation(len(b))][: (len(b) // 16) * 16].reshape(-1, 16)
    t = bf16_to_f32(b)
    S_enc, _ = R.nvfp4_tensor_scales(R.amax(t))
    r = philox_word_for_index(np.arange(t.size), 42).reshape(t.shape)
    for sr in (False, True):
        packed, d = R.quantize_nvfp4(t, S_enc, sr_random=r if sr else None)
        codes = R.unpack_e2m1(packed)
        for i in range(0, t.shape[0], 3):
            a_b = max(abs(Fraction(float(z))) for z in t[i])
            dv = frac_to_f32(Fraction(frac_to_f32(a_b / 6)) * Fraction(float(S_enc)))
            dc = int(_brute_e4m3(np.array([dv], np.float32))[0])
            assert d[i, 0] == dc
            dval = float(E4M3.decode(dc))
            for j in range(16):
                if dval == 0:
                    want = 8 if np.signbit(t[i, j]) else 0
                else:
                    eb = frac_to_f32(Fraction(float(S_enc)) / Fraction(dval))
                    eb = FLT_MAX if eb == math.inf else eb
                    v = np.float32(frac_to_f32(Fraction(float(t[i, j])) * Fraction(eb)))
                    if np.signbit(t[i, j]) and v == 0:
                        v = np.float32(-0.0)
                    if not sr:
                        want = _frac_nearest_e2m1(v)
                    else:
                        av = abs(Fraction(float(v)))
                        mags = [Fraction(float(m)) for m in E2M1.magnitudes]
                        if av >= 6:
                            c = 7
                        else:
                            lo = max(k for k in range(8) if mags[k] <= av)
                            P = (av - mags[lo]) / (mags[lo + 1] - mags[lo])
                            c = lo + 1 if int(r[i, j]) < P * 2 ** 32 else lo
                        want = c | (8 if np.signbit(v) else 0)
                assert codes[i, j] == want, (i, j, sr)


def test_encode_saturates_overflowed_product():
    from oracle.formats import E4M3, E5M2, E2M1
    inf = np.float32(np.inf)
    for f in (E4M3, E5M2, E2M1):
        assert f.encode(np.array([inf]))[0] == f.max_code
        assert f.encode(np.array([-inf]))[0] == f.max_code | f.sign_bit
    with pytest.raises(ValueError):
        E4M3.encode(np.array([np.nan], np.float32))
