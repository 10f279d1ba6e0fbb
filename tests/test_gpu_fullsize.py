"""Full-size parity on the benchmark's own workload.

The CodonFM-5B layer at M = 31 x 512 = 15872 tokens, hidden 4096,
intermediate 16384 ("How to optimize Transformer-based models for
low-precision training", "Model configuration and training inputs"), with
the benchmark's seeded inputs and its launch configuration (plus the same
layer at 32768 tokens and a Llama-3-8B-shaped layer at 8192): each GEMM
quantizes both operands on the GPU (autocast path of the pipeline) and runs
with bf16 output.  The oracle cannot quantize and multiply 260M-element
tensors one by one in seconds, so it checks samples it computes exactly:

* whole 128-row groups of every quantized copy (the first three, a middle
  and the last group; blocks never straddle a group), codes and scales bit
  for bit;
  per-tensor scales and the NVFP4 encode scale come from the oracle's amax
  of the whole tensor (after the Hadamard transform for NVFP4 Wgrad inputs);
* GEMM outputs at about 11 x 11 (m, n) pairs drawn from those rows (first,
  last, either side of the first 256-row tile boundary, random), against the
  fp64 dot product of the oracle-dequantized rows, within
  |err| <= 1e-5 sum|a b| (+ the 8-bit instruction's unit bound, + 1 bf16 ulp);
* the GEMM epilogue's max |C| (pbs_gemm_amax) against the amax kernel's
  pass over the whole stored C, bit for bit.
"""
import functools

import numpy as np
import pytest
import torch

import workloads as W
import precision_block_scaled_amd as P
from precision_block_scaled_amd import pipeline as PL
from oracle import recipes as R
from oracle.formats import bf16_to_f32
from oracle.gemm_ref import check_gemm, fp8_dot_unit_bound
from oracle.passes import BLOCK128_2D
from oracle.philox import philox_word0_for_index
from tests.gpu_util import to_gpu_bf16

pytestmark = pytest.mark.gpu

# model -> (tokens, layer shapes): the CodonFM-5B layer the benchmark times,
# the same layer at 32 x 1024 tokens, and a Llama-3-8B-shaped layer (GQA
# 32 q / 8 kv heads: QKV N = 6144; gated MLP: up N = 28672, down K = 14336)
# at 8192 tokens
L3 = W.LLAMA3_8B_LAYER
MODELS = {
    "codonfm": (15872, W.layer_shapes(4096, 16384, 32)),
    "codonfm_32k": (32768, W.layer_shapes(4096, 16384, 32)),
    "llama3_8b": (8192, W.layer_shapes(L3["hidden"], L3["intermediate"], L3["heads"], L3["kv_heads"],
                                       L3["gated"])),
}
FP8_MFMA = {"fp8_current", "fp8_delayed", "mxfp8", "fp8_channel", "fp8_block128_pow2"} | set(BLOCK128_2D)
FMAX = {"e4m3": 448.0, "e5m2": 57344.0}
SEED = 42


@functools.lru_cache(maxsize=2)
def layer_inputs(model, name):
    """The benchmark's tensors for one layer (seeds 10+i, 20+i, 30+i), bf16 bits."""
    tokens, shapes = MODELS[model]
    i, ls = next((i, ls) for i, ls in enumerate(shapes) if ls.name == name)
    x = W.activations(tokens, ls.k_in, seed=10 + i)
    w = W.weights(ls.n_out, ls.k_in, seed=20 + i)
    dy = W.grads(tokens, ls.n_out, seed=30 + i)
    return x, w, dy


def groups_of(n_rows):
    """The first three, a middle and the last 128-row group of a copy with
    n_rows rows (groups 1 and 2 straddle the first 256-row tile boundary)."""
    g = n_rows // 128
    return sorted({0, 1, 2, g // 2, g - 1} & set(range(g)))


def copy_rows(bits, orient, rows):
    """Rows `rows` of the copy of `bits` (source layout) in orientation `orient`, source layout slice."""
    return bits[rows, :] if orient == "row" else bits[:, rows]


class OracleCopy:
    """The oracle's quantization of whole 128-row groups of one copy."""

    def __init__(self, recipe, src, orient, bits, pass_, dstate, rows):
        self.recipe, self.rows = recipe, rows
        sl = copy_rows(bits, orient, rows)
        w2d = src in BLOCK128_2D.get(recipe, ()) or (src == "w" and recipe in ("nvfp4", "fp8_block128_pow2"))
        self.tsi = None
        self.scales = None
        if recipe in ("fp8_current", "fp8_delayed"):
            fmt = "e5m2" if src == "dy" else "e4m3"
            if recipe == "fp8_current":
                s, s_inv = R.scale_from_amax(R.amax(bits), FMAX[fmt])
                self.codes = R.cast_pertensor(sl, s, fmt, orient)
            else:
                self.codes, s_inv, _ = dstate.cast(sl, orient)
            self.tsi = np.float32(s_inv)
            self.deq = R.dequant_pertensor(self.codes, fmt, self.tsi)
        elif recipe in BLOCK128_2D:
            self.codes, self.scales = R.quantize_block128(sl, orient, weight_2d=w2d)
            self.deq = R.dequant_block128(self.codes, self.scales, w2d)
        elif recipe == "fp8_block128_pow2":             # scales compared as E8M0 codes
            self.codes, self.scales = R.quantize_block128_pow2(sl, orient, weight_2d=w2d)
            self.deq = R.dequant_block128_pow2(self.codes, self.scales, w2d)
        elif recipe == "fp8_channel":                   # a copy row's scale is its own
            self.codes, self.scales = R.quantize_channel(sl, orient)
            self.deq = R.dequant_channel(self.codes, self.scales)
        elif recipe == "mxfp8":
            self.codes, self.scales = R.quantize_mxfp8(sl, orient)
            self.deq = R.dequant_mxfp8(self.codes, self.scales)
        elif recipe in ("nvfp4", "mxfp4"):
            rht = pass_ == "wgrad"
            t = bf16_to_f32(sl)
            if rht:
                t = R.rht16_along_rows(t, SEED)          # col slices hold whole columns
            t_o = t if orient == "row" else np.ascontiguousarray(t.T)
            sr = None
            if src == "dy":
                M, N = bits.shape
                r = np.asarray(rows, dtype=np.uint64)
                if orient == "row":
                    idx = r[:, None] * np.uint64(N) + np.arange(N, dtype=np.uint64)[None, :]
                else:
                    idx = np.arange(M, dtype=np.uint64)[None, :] * np.uint64(N) + r[:, None]
                sr = philox_word0_for_index(idx, SEED)
            if recipe == "nvfp4":
                A = R.amax(R.rht16_along_rows(bf16_to_f32(bits), SEED) if rht else bits)
                S_enc, S_dec = R.nvfp4_tensor_scales(A)
                self.codes, self.scales = R.quantize_nvfp4(t_o, S_enc, weight_2d=w2d, sr_random=sr)
                self.tsi = np.float32(S_dec)
                self.deq = R.dequant_nvfp4(self.codes, self.scales, self.tsi, w2d)
            else:
                self.codes, self.scales = R.quantize_mxfp4(t_o, sr_random=sr)
                self.deq = R.dequant_mxfp4(self.codes, self.scales)
        else:  # bf16: the operand is the natural-layout tensor
            self.codes = sl if orient == "row" else np.ascontiguousarray(sl.T)
            self.deq = bf16_to_f32(self.codes).astype(np.float64)
        self.w2d = w2d


def gpu_rows(q, rows, w2d):
    """Codes and scales of the GPU copy q for whole 128-row groups `rows`."""
    idx = torch.from_numpy(np.asarray(rows, dtype=np.int64)).to(q.codes.device)
    codes = q.codes[idx].cpu().numpy()
    sc = None
    if q.scales is not None:
        if w2d:
            div = 128 if q.recipe in BLOCK128_2D or q.recipe == "fp8_block128_pow2" else 16
            g = torch.from_numpy(np.unique(np.asarray(rows) // div).astype(np.int64)).to(q.codes.device)
            sc = q.scales[g].cpu().numpy()
        else:
            sc = q.scales[idx].cpu().numpy()
    return codes, sc


def run_pass(recipe, model, name, pass_):
    x, w, dy = layer_inputs(model, name)
    src = {"x": x, "w": w, "dy": dy}
    dev = "cuda"
    xg, wg, dyg = to_gpu_bf16(x), to_gpu_bf16(w), to_gpu_bf16(dy)
    M, N, K = PL.pass_dims(pass_, x.shape[0], x.shape[1], w.shape[0])
    states, ostates = None, {}
    if recipe == "fp8_delayed":
        # one earlier step: each history holds the tensor's own amax
        states = {k: PL.DelayedState(P.PBS_FMT_E5M2 if k == "dy" else P.PBS_FMT_E4M3, dev)
                  for k in ("x", "w", "dy")}
        for k, t in (("x", xg), ("w", wg), ("dy", dyg)):
            P.pbs_amax(t, t.shape[0], t.shape[1], 0, 0, states[k].amax)
            states[k].update()
        for k in ("x", "w", "dy"):
            ostates[k] = R.DelayedScaling("e5m2" if k == "dy" else "e4m3")
            ostates[k].update(R.amax(src[k]))
    if recipe == "bf16":
        A, B = {"fprop": (xg, wg), "dgrad": (dyg, wg), "wgrad": (xg, dyg)}[pass_]
    else:
        A, B = PL.quantize_pass(recipe, pass_, xg, wg, dyg, states=states)
    c_amax = torch.full((1,), -1.0, device=dev)
    C = PL.gemm(recipe, pass_, A, B, M, N, K, out_dtype=torch.bfloat16, c_amax=c_amax)
    full_amax = torch.zeros(1, device=dev)
    P.pbs_amax(C, M, N, 0, 0, full_amax)
    torch.cuda.synchronize()

    from oracle.passes import operand_roles
    (sa, oa), (sb, ob) = operand_roles(pass_)
    if recipe == "bf16":
        oa, ob = {"fprop": ("row", "row"), "dgrad": ("row", "col"), "wgrad": ("col", "col")}[pass_]
    out = []
    rows_a = np.concatenate([np.arange(128 * g, 128 * g + 128) for g in groups_of(M)])
    rows_b = np.concatenate([np.arange(128 * g, 128 * g + 128) for g in groups_of(N)])
    qa = OracleCopy(recipe, sa, oa, src[sa], pass_, ostates.get(sa), rows_a)
    qb = OracleCopy(recipe, sb, ob, src[sb], pass_, ostates.get(sb), rows_b)
    if recipe != "bf16":
        for q, o, rows, sname in ((A, qa, rows_a, sa), (B, qb, rows_b, sb)):
            codes, sc = gpu_rows(q, rows, o.w2d)
            if (codes != o.codes).any():
                i = tuple(np.argwhere(codes != o.codes)[0])
                out.append(f"codes differ at sampled {i}: {codes[i]} vs {o.codes[i]}")
            if recipe == "fp8_block128_pow2":            # each word: the E8M0 code in all four bytes
                if (sc.view(np.uint32) != o.scales.astype(np.uint32) * np.uint32(0x01010101)).any():
                    out.append("block scale words differ")
            elif o.scales is not None and (sc.view(np.uint8) != np.ascontiguousarray(o.scales).view(np.uint8)).any():
                out.append("block scales differ")
            if o.tsi is not None:
                if isinstance(q.tensor_scale_inv, int):   # delayed: the state's scale_inv word
                    g_tsi = states[sname].buf[4:8].cpu().numpy().view(np.float32)[0]
                else:
                    g_tsi = q.tensor_scale_inv.cpu().numpy()[0]
                if np.float32(g_tsi).view(np.uint32) != np.float32(o.tsi).view(np.uint32):
                    out.append(f"tensor scale_inv {g_tsi} vs {o.tsi}")
    # the epilogue's max |C| equals the amax kernel's pass over the stored C
    if c_amax.cpu().numpy().view(np.uint32)[0] != full_amax.cpu().numpy().view(np.uint32)[0]:
        out.append(f"epilogue amax {c_amax.item()} vs amax of C {full_amax.item()}")
    rng = np.random.default_rng(7)
    # first and last rows, rows 255 / 256 / 257 (either side of the first 256-row tile boundary), random rows
    edge_a = [int(np.searchsorted(rows_a, r)) for r in (255, 256, 257)]
    edge_b = [int(np.searchsorted(rows_b, r)) for r in (255, 256, 257)]
    ia = np.unique(np.concatenate([[0, len(rows_a) - 1], edge_a, rng.choice(len(rows_a), 6, replace=False)]))
    ib = np.unique(np.concatenate([[0, len(rows_b) - 1], edge_b, rng.choice(len(rows_b), 6, replace=False)]))
    ah, bh = qa.deq[ia], qb.deq[ib]
    cref = ah @ bh.T
    bnd = np.abs(ah) @ np.abs(bh).T
    extra = fp8_dot_unit_bound(ah, bh) if recipe in FP8_MFMA else None
    c = C[torch.from_numpy(rows_a[ia]).cuda()][:, torch.from_numpy(rows_b[ib]).cuda()]
    c = c.float().cpu().numpy()
    ok, tol, err = check_gemm(c, cref, bnd, True, extra)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        out.append(f"GEMM {(~ok).sum()} of {ok.size} outside bound; got {c[i]} want {cref[i]} tol {tol[i]}")
    return out


RECIPES = ["bf16", "fp8_current", "fp8_delayed", "fp8_block128", "mxfp8", "nvfp4"]
CASES = ([("codonfm", n, r) for n in ("qkv", "attn_out", "mlp_up", "mlp_down") for r in RECIPES]
         + [("llama3_8b", n, r) for n in ("qkv", "attn_out", "mlp_up", "mlp_down") for r in RECIPES]
         + [("codonfm_32k", n, r) for n in ("mlp_up", "mlp_down") for r in ("mxfp8", "nvfp4", "fp8_block128")]
         + [(m, n, r) for r in ("mxfp4", "fp8_channel") for m in ("codonfm", "llama3_8b")
            for n in ("qkv", "attn_out", "mlp_up", "mlp_down")]
         + [("codonfm", n, r) for r in ("fp8_block128_1d1d", "fp8_block128_2d2d")
            for n in ("qkv", "attn_out", "mlp_up", "mlp_down")]
         + [(m, n, "fp8_block128_pow2") for m in ("codonfm", "llama3_8b")
            for n in ("qkv", "attn_out", "mlp_up", "mlp_down")])


@pytest.mark.parametrize("model,name,recipe", CASES)
def test_fullsize_layer(model, name, recipe):
    problems = []
    for pass_ in ("fprop", "dgrad", "wgrad"):
        problems += [f"{pass_}: {p}" for p in run_pass(recipe, model, name, pass_)]
    assert not problems, f"{model} {name} {recipe}: " + "; ".join(problems)
