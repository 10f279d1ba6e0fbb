"""NVFP4 casts at their edges, bit for bit against the oracle.

NVFP4 ("Accelerate LLM training with NVFP4 on Blackwell", "Technical
deep-dive": E2M1 values, one E4M3 scale per 16 values and one fp32 scale per
tensor; "How to optimize Transformer-based models for low-precision
training", "Interpreting results for a real model": 16x16 weight blocks,
the Hadamard transform on the Wgrad inputs, stochastic rounding of
gradients) has the most intricate arithmetic of the recipes: a block scale
that is itself rounded to E4M3, an encode factor S_enc / d that can
overflow, and blocks whose scale rounds to zero.  Every kernel variant
(row copy, col copy, both copies from one read, 16x16 weight blocks, the
Hadamard col copy, with and without stochastic rounding) runs on:

* all 65,536 bf16 bit patterns (non-finite ones zeroed), as a [256, 256]
  tensor, under several encode scales S_enc: the tensor's own
  fp32(2688 / amax), 1, 2**-60, 2**60 and FLT_MAX (where S_enc / d
  overflows to FLT_MAX on the subnormal blocks);
* planted blocks: all zero, all -0, a block scale that rounds to zero (a tie
  at half the smallest E4M3 subnormal), E4M3 block-scale ties either way,
  E2M1 value ties, bf16 subnormals, mixed signs.
"""
import numpy as np
import pytest
import torch

import workloads as W
import precision_block_scaled_amd as P
from oracle import recipes as R
from oracle.formats import bf16_to_f32
from tests.gpu_util import first_mismatch, scalar_gpu, to_gpu_bf16, to_np_u8

pytestmark = pytest.mark.gpu

FLT_MAX = np.float32(3.4028234663852886e38)
SEED = 42


def _cast(x_bits, S_enc, orient_mask, w2d=False, flags=0):
    """GPU NVFP4 cast of x [R, C]: (row codes, row scales, col codes, col scales)."""
    Rr, Cc = x_bits.shape
    row = orient_mask & P.PBS_ROW
    col = orient_mask & P.PBS_COL
    rc = torch.empty((Rr, Cc // 2), dtype=torch.uint8, device="cuda") if row else None
    cc = torch.empty((Cc, Rr // 2), dtype=torch.uint8, device="cuda") if col else None
    if w2d:
        rs = torch.empty((Rr // 16, Cc // 16), dtype=torch.uint8, device="cuda") if row else None
        cs = torch.empty((Cc // 16, Rr // 16), dtype=torch.uint8, device="cuda") if col else None
    else:
        rs = torch.empty((Rr, Cc // 16), dtype=torch.uint8, device="cuda") if row else None
        cs = torch.empty((Cc, Rr // 16), dtype=torch.uint8, device="cuda") if col else None
    P.pbs_cast(P.PBS_RECIPE_NVFP4, to_gpu_bf16(x_bits), Rr, Cc, P.PBS_FMT_E2M1, orient_mask, int(w2d), flags, SEED,
               scalar_gpu(S_enc), None, rc, rs, cc, cs)
    torch.cuda.synchronize()
    return tuple(to_np_u8(t) if t is not None else None for t in (rc, rs, cc, cs))


def _oracle(x_bits, S_enc, orient, w2d=False, rht=False, sr=False):
    t = bf16_to_f32(x_bits)
    if rht:
        t = R.rht16_along_rows(t, SEED)
    t_o = t if orient == "row" else np.ascontiguousarray(t.T)
    rnd = R.sr_random_for(x_bits.shape, orient, SEED) if sr else None
    return R.quantize_nvfp4(t_o, np.float32(S_enc), weight_2d=w2d, sr_random=rnd)


def _check(got_codes, got_scales, want, what):
    wc, ws = want
    assert first_mismatch(got_scales, ws) is None, f"{what}: block scales {first_mismatch(got_scales, ws)}"
    assert first_mismatch(got_codes, wc) is None, f"{what}: codes {first_mismatch(got_codes, wc)}"


def _all_patterns(limit_exponent=None):
    x = W.all_bf16_patterns()
    if limit_exponent is not None:      # the Hadamard sums of 16 huge values overflow fp32
        e = (x >> 7) & 0xFF
        x = np.where(e >= limit_exponent, np.uint16(0), x).astype(np.uint16)
    return x


def _scales_for(x_bits, rht=False):
    t = bf16_to_f32(x_bits)
    if rht:
        t = R.rht16_along_rows(t, SEED)
    own = R.nvfp4_tensor_scales(R.amax(t))[0]
    return [own, np.float32(1.0), np.float32(2.0 ** -60), np.float32(2.0 ** 60), FLT_MAX]


VARIANTS = [  # (orient mask, w2d, flags) -- every kernel the NVFP4 casts select
    (P.PBS_ROW, False, 0), (P.PBS_ROW, False, P.PBS_FLAG_SR),
    (P.PBS_COL, False, 0), (P.PBS_COL, False, P.PBS_FLAG_SR),
    (P.PBS_ROW | P.PBS_COL, False, 0), (P.PBS_ROW | P.PBS_COL, False, P.PBS_FLAG_SR),
    (P.PBS_ROW, True, 0), (P.PBS_COL, True, 0), (P.PBS_ROW | P.PBS_COL, True, 0),
    (P.PBS_COL, False, P.PBS_FLAG_RHT16), (P.PBS_COL, False, P.PBS_FLAG_RHT16 | P.PBS_FLAG_SR),
]


def _run_variant(x, mask, w2d, flags, S_list=None):
    rht = bool(flags & P.PBS_FLAG_RHT16)
    sr = bool(flags & P.PBS_FLAG_SR)
    for S in (S_list if S_list is not None else _scales_for(x, rht)):
        rc, rs, cc, cs = _cast(x, S, mask, w2d, flags)
        if mask & P.PBS_ROW:
            _check(rc, rs, _oracle(x, S, "row", w2d, False, sr), f"row S={S!r} w2d={w2d} flags={flags}")
        if mask & P.PBS_COL:
            _check(cc, cs, _oracle(x, S, "col", w2d, rht, sr), f"col S={S!r} w2d={w2d} flags={flags}")


@pytest.mark.parametrize("mask,w2d,flags", VARIANTS)
def test_all_bf16_patterns(mask, w2d, flags):
    rht = bool(flags & P.PBS_FLAG_RHT16)
    _run_variant(_all_patterns(0xF8 if rht else None), mask, w2d, flags)


def planted_blocks():
    """16-value blocks (float32, exact bf16 values) for the edge cases."""
    blocks = []
    blocks.append(np.zeros(16, np.float32))                           # all +0: d = 0
    blocks.append(np.full(16, -0.0, np.float32))                      # all -0: codes 0x8
    z = np.zeros(16, np.float32)
    z[3] = np.float32(6 * 2.0 ** -10)                                 # a_b / 6 = 2**-10: tie -> d = 0
    z[4] = -np.float32(2.0 ** -12)
    z[5] = -0.0
    blocks.append(z)
    t = np.zeros(16, np.float32)
    t[0] = np.float32(6 * 3 * 2.0 ** -10)                             # d tie between codes 1 and 2 -> 2
    t[1:8] = np.float32(2.0 ** -9)
    blocks.append(t)
    for m in (6.375, 7.125, 6.75, 13.5):                              # block-scale ties / near ties at S_enc 1
        b = np.linspace(-m, m, 16).astype(np.float32)
        b = bf16_to_f32(W.f32_to_bf16_bits(b))
        b[0] = np.float32(-m)
        blocks.append(b)
    v = np.array([6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5, -6],
                 np.float32)                                          # E2M1 ties with d = 1 at S_enc 1
    blocks.append(v)
    blocks.append(-v)
    sub = (np.arange(16, dtype=np.uint32) * 7 + 1).astype(np.uint16)  # bf16 subnormals
    blocks.append(bf16_to_f32(sub))
    blocks.append(-bf16_to_f32(sub))
    mixed = np.array([1e-30, -3e-20, 2.0, -448.0, 1e10, -1e-38, 5.5, -0.0, 0.0, 1.0, -1.0, 3.0, -3.0, 0.5, 64.0,
                      -64.0], np.float32)
    blocks.append(bf16_to_f32(W.f32_to_bf16_bits(mixed)))
    return [bf16_to_f32(W.f32_to_bf16_bits(b)) for b in blocks]


def planted_tensor(seed=3):
    """[16, 256] bf16 bits: the planted blocks first along the rows (row r
    holds blocks 16 r .. 16 r + 15), random bf16 values after them."""
    blocks = planted_blocks()
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((16, 256)) * rng.choice([1e-3, 1.0, 100.0], size=(16, 256))).astype(np.float32)
    for i, b in enumerate(blocks):
        r, c = divmod(i, 16)
        x[r, 16 * c:16 * c + 16] = b
    return W.f32_to_bf16_bits(x)


@pytest.mark.parametrize("mask,w2d,flags", [v for v in VARIANTS if not v[1]])
def test_planted_blocks_1d(mask, w2d, flags):
    """Row and two-copy variants take the planted tensor as is, the col
    variants its transpose, so that the planted blocks run down the columns."""
    x = planted_tensor()
    if mask == P.PBS_COL:
        x = np.ascontiguousarray(x.T)
    S_list = [np.float32(1.0), np.float32(6.0), np.float32(2688.0 / 448.0), FLT_MAX]
    if flags & P.PBS_FLAG_RHT16:
        S_list.append(R.nvfp4_tensor_scales(R.amax(R.rht16_along_rows(bf16_to_f32(x), SEED)))[0])
    _run_variant(x, mask, w2d, flags, S_list)


@pytest.mark.parametrize("mask", [P.PBS_ROW, P.PBS_COL, P.PBS_ROW | P.PBS_COL])
def test_planted_blocks_2d(mask):
    """16x16 weight blocks: each planted block repeated down its 16 rows,
    alternate rows negated, so the 2D maximum is the block's maximum."""
    blocks = planted_blocks()
    x = np.zeros((16, 16 * len(blocks)), np.float32)
    for i, b in enumerate(blocks):
        for r in range(16):
            x[r, 16 * i:16 * i + 16] = b if r % 2 == 0 else -b
    xb = W.f32_to_bf16_bits(x)
    _run_variant(xb, mask, True, 0, [np.float32(1.0), np.float32(6.0), FLT_MAX])


def test_rht_cast_entry_point_seeds():
    """pbs_rht_cast keys the Hadamard signs and the stochastic rounding with
    separate seeds; with equal seeds it is pbs_cast's Hadamard col copy."""
    x = W.grads(256, 96, seed=17)
    t = bf16_to_f32(x)
    for recipe in ("nvfp4", "mxfp4"):
        for rht_seed, sr_seed, sto in ((42, 42, 1), (7, 1234567, 1), (99, 0, 0)):
            ty = R.rht16_along_rows(t, rht_seed)
            tt = np.ascontiguousarray(ty.T)
            rnd = R.sr_random_for(x.shape, "col", sr_seed) if sto else None
            cc = torch.empty((96, 128), dtype=torch.uint8, device="cuda")
            if recipe == "nvfp4":
                S = R.nvfp4_tensor_scales(R.amax(ty))[0]
                want = R.quantize_nvfp4(tt, S, sr_random=rnd)
                cs = torch.empty((96, 16), dtype=torch.uint8, device="cuda")
                P.pbs_rht_cast(P.PBS_RECIPE_NVFP4, to_gpu_bf16(x), 256, 96, rht_seed, sto, sr_seed, scalar_gpu(S),
                               cc, cs)
            else:
                want = R.quantize_mxfp4(tt, sr_random=rnd)
                cs = torch.empty((96, 8), dtype=torch.uint8, device="cuda")
                P.pbs_rht_cast(P.PBS_RECIPE_MXFP4, to_gpu_bf16(x), 256, 96, rht_seed, sto, sr_seed, None, cc, cs)
            torch.cuda.synchronize()
            _check(to_np_u8(cc), to_np_u8(cs), want, f"{recipe} rht_seed={rht_seed} sr_seed={sr_seed} sr={sto}")
