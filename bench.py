"""Benchmark: quantize-then-GEMM over the 12 GEMMs of a Transformer layer.

Workload ("How to optimize Transformer-based models for low-precision
training", "Model configuration and training inputs" and "Using autocast
mode vs pre-quantized mode"): a model configuration (hidden size,
intermediate size, attention heads and key/value heads, gated MLP or not)
and a batch (micro-batch x sequence length tokens) give the QKV,
attention-out, MLP-up and MLP-down linear layers, each in Fprop, Dgrad and
Wgrad: 12 GEMMs.  The default is the CodonFM-5B layer: hidden 4096,
intermediate 16384, 32 heads, micro-batch 31 x sequence 512 = 15872 tokens.

One step = every recipe (BF16, FP8 current, FP8 delayed, FP8 1x128/128x128,
MXFP8, NVFP4) over the 12 GEMMs in autocast mode: each GEMM quantizes both
of its operands from bf16 (amax, scale, cast, RHT, SR as the recipe needs)
and then runs the GEMM, bf16 output.  With --pre-quantize the step times the
GEMMs alone on operands quantized beforehand.  As in the pages' tool,
--no-fp8 drops MXFP8, --no-fp4 the 4-bit recipes, --num_hidden_layers sets
the layer count of the model-level projection, and -o writes the per-GEMM
speedup-over-BF16 chart of the timed mode.  Inputs are seeded synthetic
tensors resident in HBM before timing starts; each layer has its own X, W
and dY.

Printed: one JSON line.  ``value`` = total GEMM FLOP of the step / step time
(TFLOP/s), plus per-recipe ms/layer and TFLOP/s in autocast, pre-quantized
(operands hot in the caches, and cold) and layer-autocast modes,
quantize-pass GB/s, the roofline of the dominant kernel (timed with HIP
events on the stream it runs on), the same sweep on the CodonFM layer at
32 x 1024 tokens and on a Llama-3-8B-shaped layer at 8192 tokens, and the
CPU oracle timed on a bounded sample of the workload beside the GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

RECIPES = ["bf16", "fp8_current", "fp8_delayed", "fp8_block128", "mxfp8", "nvfp4"]
# built beyond the pages' six (MXFP4: E2M1 with E8M0 per 32 on the FP4 matrix
# rate); timed after the step and reported apart, never part of `value`
NEXT_RECIPES = ["mxfp4", "fp8_channel", "fp8_block128_1d1d", "fp8_block128_2d2d", "fp8_block128_pow2"]
PEAK_TFLOPS = {"bf16": 2516.6, "fp16": 2516.6, "fp8": 5033.2, "fp4": 10066.3}
HBM_GBPS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_key(recipe, pass_):
    """The GEMM kernel instantiation a (recipe, pass) launches, and its MFMA dtype."""
    if recipe == "bf16":
        return f"gemm_bf16_{pass_}", "bf16"
    if recipe in ("fp8_current", "fp8_delayed"):
        fmts = {"fprop": "e4m3xe4m3", "dgrad": "e5m2xe4m3", "wgrad": "e4m3xe5m2"}[pass_]
        return f"gemm_fp8_tensor_{fmts}", "fp8"
    if recipe == "fp8_block128":
        return ("gemm_fp8_block128_w2d" if pass_ != "wgrad" else "gemm_fp8_block128_1d"), "fp8"
    if recipe == "mxfp8":
        return "gemm_mxfp8", "fp8"
    if recipe == "mxfp4":
        return "gemm_mxfp4", "fp4"
    if recipe == "fp8_channel":
        return "gemm_fp8_channel", "fp8"
    if recipe == "fp8_block128_1d1d":
        return "gemm_fp8_block128_1d", "fp8"
    if recipe == "fp8_block128_2d2d":
        return "gemm_fp8_block128_2d2d", "fp8"
    if recipe == "fp8_block128_pow2":
        return "gemm_fp8_block128_pow2", "fp8"
    return ("gemm_nvfp4_w2d" if pass_ != "wgrad" else "gemm_nvfp4_1d"), "fp16"


# the sources each kernel family is built from: its HBM counters stay valid
# while these files are unchanged
KERNEL_SOURCES = {    # first matching prefix wins
    "gemm_fp8_block128": ("gemm.hip", "gemm_blk.hip", "gemm_common.hpp", "device.hpp", "host.hpp"),
    "gemm_": ("gemm.hip", "gemm_common.hpp", "device.hpp", "host.hpp"),
    "cast_": ("cast.hip", "device.hpp", "host.hpp"),
    "chan_": ("cast.hip", "device.hpp", "host.hpp"),
    "amax": ("amax.hip", "device.hpp", "host.hpp"),
}


def kernel_source_files(kernel_name):
    for prefix, files in KERNEL_SOURCES.items():
        if kernel_name.startswith(prefix):
            return files
    return tuple(sorted(os.listdir(os.path.join(ROOT, "precision_block_scaled_amd", "csrc"))))


def source_digest(files=None):
    """Digest of the HIP sources `files` (default: all of them)."""
    d = os.path.join(ROOT, "precision_block_scaled_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(files if files is not None else os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def upload_bf16(bits, dev):
    import torch
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)


# model configurations: the pages' CodonFM-5B layer, and a Llama-3-8B-shaped
# layer (GQA 32 query / 8 key-value heads, gated MLP)
MODELS = {
    "codonfm": dict(hidden=4096, intermediate=16384, heads=32, kv_heads=32, gated=False, micro_batch=31,
                    seq_len=512, num_layers=24),
    "llama3_8b": dict(hidden=4096, intermediate=14336, heads=32, kv_heads=8, gated=True, micro_batch=1,
                      seq_len=8192, num_layers=32),
}


def build_layer_tensors(cfg, tokens, dev):
    import workloads as W
    layers = {}
    shapes = W.layer_shapes(cfg["hidden"], cfg["intermediate"], cfg["heads"], cfg["kv_heads"], cfg["gated"])
    for i, ls in enumerate(shapes):
        x = upload_bf16(W.activations(tokens, ls.k_in, seed=10 + i), dev)
        w = upload_bf16(W.weights(ls.n_out, ls.k_in, seed=20 + i), dev)
        dy = upload_bf16(W.grads(tokens, ls.n_out, seed=30 + i), dev)
        layers[ls.name] = (x, w, dy, ls)
    return layers


class Runner:
    """Holds pre-allocated quantized operands and outputs for every (recipe, GEMM)."""

    def __init__(self, layers, tokens, dev):
        import torch
        from precision_block_scaled_amd import pipeline as PL
        import precision_block_scaled_amd as P
        self.torch, self.PL, self.P = torch, PL, P
        self.layers = layers
        self.tokens = tokens
        self.dev = dev
        self.gemms = []          # (layer, pass, M, N, K)
        for name, (x, w, dy, ls) in layers.items():
            for p in ("fprop", "dgrad", "wgrad"):
                M, N, K = PL.pass_dims(p, tokens, ls.k_in, ls.n_out)
                self.gemms.append((name, p, M, N, K))
        self.C = {}
        for (name, p, M, N, K) in self.gemms:
            self.C[(name, p)] = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        self.q = {}              # (recipe, layer, pass) -> (A, B)
        self.states = {}         # delayed states per (layer, src)
        for name, (x, w, dy, ls) in layers.items():
            for src, fmt in (("x", P.PBS_FMT_E4M3), ("w", P.PBS_FMT_E4M3), ("dy", P.PBS_FMT_E5M2)):
                self.states[(name, src)] = PL.DelayedState(fmt, dev)

    def operands(self, recipe, name, p):
        PL = self.PL
        x, w, dy, ls = self.layers[name]
        src = {"x": x, "w": w, "dy": dy}
        (sa, oa), (sb, ob) = PL.ROLES[p]
        if recipe == "bf16":
            return src[sa], src[sb], None
        st = {k: self.states[(name, k)] for k in ("x", "w", "dy")} if recipe == "fp8_delayed" else {}
        prev = self.q.get((recipe, name, p))
        A = PL.quantize(recipe, src[sa], sa, oa, p, st.get(sa), prev[0] if prev else None)
        B = PL.quantize(recipe, src[sb], sb, ob, p, st.get(sb), prev[1] if prev else None)
        self.q[(recipe, name, p)] = (A, B)
        return A, B, (st.get(sa), st.get(sb))

    def run_gemm(self, recipe, name, p, A, B, M, N, K):
        self.PL.gemm(recipe, p, A, B, M, N, K, C=self.C[(name, p)])

    def step(self, recipes, events=None):
        """One autocast pass over all recipes x 12 GEMMs.  events: list to append timing.

        Delayed scaling: every GEMM casts with the state's scale and measures
        amax in the same pass; each tensor's state is updated once per step,
        after its last consumer (the scale of a step comes from earlier steps)."""
        torch = self.torch
        for r in recipes:
            for (name, p, M, N, K) in self.gemms:
                if events is not None:
                    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
                    e0.record()
                A, B, st = self.operands(r, name, p)
                if events is not None:
                    e1.record()
                self.run_gemm(r, name, p, A, B, M, N, K)
                if events is not None:
                    e2.record()
                    events.append((r, name, p, M, N, K, e0, e1, e2))
            if r == "fp8_delayed":
                for s in self.states.values():
                    s.update()

    def gemm_step(self, recipes, events):
        """One pre-quantized pass: the 12 GEMMs of every recipe on the operands
        the last autocast step quantized (events as in step, e0 == e1)."""
        torch = self.torch
        for r in recipes:
            for (name, p, M, N, K) in self.gemms:
                A, B = (self.operands(r, name, p)[:2] if r == "bf16" else self.q[(r, name, p)])
                e0, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
                e0.record()
                self.run_gemm(r, name, p, A, B, M, N, K)
                e2.record()
                events.append((r, name, p, M, N, K, e0, e0, e2))

    def prequant_pass(self, recipes, iters, cold=False):
        """GEMM-only timing with operands quantized once beforehand: {(recipe,
        layer, pass): (median ms, min ms)}.  Back to back, an operand that fits
        the 256 MB last-level cache stays there; with `cold` a 1 GiB scratch
        write between iterations (outside the events) evicts it first."""
        torch = self.torch
        out = {}
        scratch = torch.empty(1 << 28, dtype=torch.float32, device=self.dev) if cold else None
        for r in recipes:
            for (name, p, M, N, K) in self.gemms:
                if r == "bf16":
                    A, B, _ = self.operands(r, name, p)
                else:
                    A, B = self.q[(r, name, p)]
                ts = []
                for _ in range(iters):
                    if cold:
                        scratch.zero_()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    self.run_gemm(r, name, p, A, B, M, N, K)
                    e1.record()
                    ts.append((e0, e1))
                out[(r, name, p)] = ts
        torch.cuda.synchronize()
        res = {}
        for k, v in out.items():
            t = [a.elapsed_time(b) for a, b in v]
            res[k] = (float(np.median(t)), float(np.min(t)))
        return res

    def layer_step(self, recipes, events, producer_amax=True):
        """Layer autocast: each of X, W and dY is quantized once per layer --
        both copies from one read wherever the two copies get the same
        treatment -- and then the layer's three GEMMs run.  With
        `producer_amax` the per-tensor maxima of X and dY come from the
        epilogue of the GEMMs that produce them (pbs_gemm_amax: each layer's
        Fprop and Dgrad fold max |C| into their epilogue for the next and the
        previous layer), so current scaling and NVFP4 read X and dY once
        (the maximum of the Hadamard-transformed tensors still takes a pass).
        events: appends (recipe, layer, ms-event pair)."""
        torch, PL, P = self.torch, self.PL, self.P
        for r in recipes:
            for name, (x, w, dy, ls) in self.layers.items():
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                cp = self.lq.get((r, name))
                st = {k: self.states[(name, k)] for k in ("x", "w", "dy")}
                known = self.known_amax[name] if producer_amax and r in ("fp8_current", "nvfp4") else {}
                amx = self.c_amax if r in ("fp8_current", "nvfp4") else None
                if r == "bf16":
                    q = {("x", "row"): x, ("w", "row"): w, ("dy", "row"): dy}
                else:
                    q = {} if cp is None else cp
                    for s_, t in (("x", x), ("w", w), ("dy", dy)):
                        if r in ("nvfp4", "mxfp4") and s_ != "w":
                            pr = "fprop" if s_ == "x" else "dgrad"
                            q[(s_, "row")] = PL.quantize(r, t, s_, "row", pr, st[s_], q.get((s_, "row")),
                                                         known_amax=known.get(s_))
                            q[(s_, "col")] = PL.quantize(r, t, s_, "col", "wgrad", st[s_], q.get((s_, "col")))
                        else:
                            prev = (q[(s_, "row")], q[(s_, "col")]) if (s_, "row") in q else None
                            q[(s_, "row")], q[(s_, "col")] = PL.quantize_both(r, t, s_, st[s_], prev,
                                                                             known_amax=known.get(s_))
                    self.lq[(r, name)] = q
                for (n_, p, M, N, K) in self.gemms:
                    if n_ != name:
                        continue
                    if r == "bf16":
                        A, B = {"fprop": (x, w), "dgrad": (dy, w), "wgrad": (x, dy)}[p]
                    else:
                        (sa, oa), (sb, ob) = PL.ROLES[p]
                        A, B = q[(sa, oa)], q[(sb, ob)]
                    PL.gemm(r, p, A, B, M, N, K, C=self.C[(name, p)],
                            c_amax=amx if (amx is not None and p != "wgrad") else None)
                e1.record()
                events.append((r, name, e0, e1))
                if r == "fp8_delayed":
                    for s_ in ("x", "w", "dy"):
                        st[s_].update()

    def prepare_layer_mode(self):
        """Buffers of the layer mode, and the maxima of X and dY that the
        producing GEMMs' epilogues would hand over (measured once, untimed)."""
        torch, P = self.torch, self.P
        self.lq = {}
        self.c_amax = torch.zeros(1, device=self.dev)
        self.known_amax = {}
        for name, (x, w, dy, ls) in self.layers.items():
            ka = {}
            for s_, t in (("x", x), ("dy", dy)):
                a = torch.zeros(1, device=self.dev)
                P.pbs_amax(t, t.shape[0], t.shape[1], 0, 0, a)
                ka[s_] = a
            self.known_amax[name] = ka
        torch.cuda.synchronize()


def quant_bandwidth(runner, iters=20):
    """GB/s of single cast passes on full-size operands (algorithmic bytes)."""
    torch, PL = runner.torch, runner.PL
    # X of MLP-down and dY of MLP-up: [15872, 16384] each, 520 MB, twice the
    # 256 MB last-level cache, so repeated casts still stream from HBM
    x = runner.layers["mlp_down"][0]
    dy = runner.layers["mlp_up"][2]
    n = x.numel()
    cases = [  # (label, recipe, src, orient, pass, algorithmic bytes per element)
        ("fp8_tensor_cast_row", "fp8_current", "x", "row", "fprop", 3.0),
        ("fp8_block128_cast_row", "fp8_block128", "x", "row", "fprop", 2 + 1 + 4 / 128),
        ("mxfp8_cast_row", "mxfp8", "x", "row", "fprop", 2 + 1 + 1 / 32),
        ("mxfp8_cast_col", "mxfp8", "x", "col", "wgrad", 2 + 1 + 1 / 32),
        ("nvfp4_cast_row", "nvfp4", "x", "row", "fprop", 2 + 0.5 + 1 / 16),
        ("nvfp4_rht_sr_cast_col", "nvfp4", "dy", "col", "wgrad", 2 + 0.5 + 1 / 16),
        ("mxfp4_cast_row", "mxfp4", "x", "row", "fprop", 2 + 0.5 + 1 / 32),
        ("mxfp4_rht_sr_cast_col", "mxfp4", "dy", "col", "wgrad", 2 + 0.5 + 1 / 32),
        # one fp32 scale per 16384-long row (row copy) / 15872-long column (col
        # copy); the col copy reads x twice (column maxima, then the cast)
        ("fp8_channel_cast_row", "fp8_channel", "x", "row", "fprop", 2 + 1 + 4 / 16384),
        ("fp8_channel_cast_col", "fp8_channel", "x", "col", "wgrad", 2 + 1 + 4 / 15872),
        # both copies from one read (the layer-autocast casts): bf16 read once,
        # two copies written
        ("fp8_tensor_cast_rowcol", "fp8_current", "x", "both", "fprop", 2 + 2 * 1.0),
        ("fp8_block128_cast_rowcol", "fp8_block128", "x", "both", "fprop", 2 + 2 * (1 + 4 / 128)),
        ("mxfp8_cast_rowcol", "mxfp8", "x", "both", "fprop", 2 + 2 * (1 + 1 / 32)),
        ("fp8_tensor_cast_col", "fp8_current", "x", "col", "wgrad", 3.0),
    ]
    res = {}
    P = runner.P

    def batch_ms(run):
        # back-to-back passes between one pair of events: the host enqueues
        # ahead of the GPU, so launch latency is not counted as pass time
        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            run()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    amax = torch.zeros(4, device=runner.dev)
    ms = batch_ms(lambda: P.pbs_amax(x, x.shape[0], x.shape[1], 0, 0, amax[0:1]))
    res["amax"] = {"ms": round(ms, 4), "GBps": round(2.0 * n / ms / 1e6, 1)}
    for label, r, src, orient, p, bpe in cases:
        t = {"x": x, "dy": dy}[src]
        rows, cols = t.shape
        rec = PL.RECIPES[r]
        if orient == "both":
            rq, cq = PL.quantize_both(r, t, src)    # allocate + warm
            out = rq
            rmask = P.PBS_ROW | P.PBS_COL
            rc, rs, cc, cs = rq.codes, rq.scales, cq.codes, cq.scales
        else:
            out = PL.quantize(r, t, src, orient, p)    # allocate + warm
            rmask = P.PBS_ROW if orient == "row" else P.PBS_COL
            rc, rs, cc, cs = ((out.codes, out.scales, None, None) if orient == "row"
                              else (None, None, out.codes, out.scales))
        flags = 0
        scale = None
        if r in ("nvfp4", "mxfp4"):
            flags = (P.PBS_FLAG_RHT16 if p == "wgrad" else 0) | (P.PBS_FLAG_SR if src == "dy" else 0)
            scale = out._scal[1:2] if r == "nvfp4" else None
        elif r == "fp8_current":
            scale = out._scal[1:2]
        ms = batch_ms(lambda: P.pbs_cast(rec, t, rows, cols, PL.fmt_for(r, src), rmask, 0, flags, 42, scale,
                                         None, rc, rs, cc, cs))
        res[label] = {"ms": round(ms, 4), "GBps": round(bpe * t.numel() / ms / 1e6, 1)}
    return res


class ClockSampler:
    """Shader clock (MHz) of the GPU, read every 20 ms from the driver's
    pp_dpm_sclk (the level marked '*'; 'S:' is the current fine-grained
    clock) while the benchmark's GEMM-heavy phases run.  None where the file
    is not readable."""

    def __init__(self, period=0.02):
        import glob
        import threading
        files = sorted(glob.glob("/sys/class/drm/card[0-9]*/device/pp_dpm_sclk"))
        self.path = files[0] if len(files) == 1 else None     # one GPU per box: no guessing among several
        self.period = period
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True) if self.path else None

    def _read(self):
        import re
        try:
            with open(self.path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        m = re.search(r"(\d+)\s*Mhz", line, re.IGNORECASE)
                        return int(m.group(1)) if m else None
        except OSError:
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        if self._thread:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread:
            self._thread.join(timeout=10)

    def summary(self):
        if not self.samples:
            return None
        v = sorted(self.samples)
        return {"sclk_MHz_min": v[0], "sclk_MHz_median": v[len(v) // 2], "sclk_MHz_max": v[-1],
                "samples": len(v), "source": f"{self.path}, every 20 ms from warm-up to the pre-quantized pass"}


def epilogue_amax_cost(runner, recipe="fp8_current", name="mlp_up", p="fprop", iters=10):
    """One GEMM with and without the epilogue max |C| (pbs_gemm_amax), beside
    the amax pass over C that it replaces."""
    torch, PL, P = runner.torch, runner.PL, runner.P
    A, B = runner.q[(recipe, name, p)]
    M, N, K = next((M, N, K) for (n, pp, M, N, K) in runner.gemms if n == name and pp == p)
    C = runner.C[(name, p)]
    amax = torch.zeros(1, device=runner.dev)

    def batch_ms(run):
        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            run()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    plain = batch_ms(lambda: PL.gemm(recipe, p, A, B, M, N, K, C=C))
    fused = batch_ms(lambda: PL.gemm(recipe, p, A, B, M, N, K, C=C, c_amax=amax))
    pass_ = batch_ms(lambda: P.pbs_amax(C, M, N, 0, 0, amax))
    return {"gemm": f"{recipe} {name}.{p} [{M}x{K}]x[{K}x{N}], bf16 out", "gemm_ms": round(plain, 4),
            "gemm_with_amax_ms": round(fused, 4), "separate_amax_pass_ms": round(pass_, 4)}


def per_gemm_times(events):
    """Per-(recipe, layer, pass) autocast and in-step GEMM times, and per-kernel totals."""
    per = {}
    for (r, name, p, M, N, K, e0, e1, e2) in events:
        d = per.setdefault((r, name, p), {"auto": [], "gemm": [], "flop": 2.0 * M * N * K})
        d["auto"].append(e0.elapsed_time(e2))
        d["gemm"].append(e1.elapsed_time(e2))
    kern = {}
    for (r, name, p), d in per.items():
        key, dt = kernel_key(r, p)
        k = kern.setdefault(key, {"ms": 0.0, "flop": 0.0, "launches": 0, "dtype": dt})
        k["ms"] += float(np.sum(d["gemm"]))
        k["flop"] += d["flop"] * len(d["gemm"])
        k["launches"] += len(d["gemm"])
    return per, kern


# matrix peak (TFLOP/s) of the instruction each recipe's GEMM runs on; exact
# NVFP4 runs on the fp16 MFMA
RECIPE_PEAK = {"bf16": 2516.6, "nvfp4": 2516.6, "mxfp4": 10066.3}
# the format's own dense peak where it differs from the instruction's: NVFP4
# is a 4-bit format (FP4 matrix rate), though its exact path issues fp16 MFMAs
FORMAT_PEAK = {"nvfp4": 10066.3}


def quant_bytes_per_element(recipe, src, k_len):
    """Algorithmic HBM bytes per element to quantize one operand in autocast:
    the bf16 read (twice when an amax pass must precede the cast), the codes
    and the block scales written.  `src` is 'x', 'w' or 'dy'; `k_len` the
    length of the copy's rows (channel scales)."""
    w2d = src == "w"
    if recipe == "bf16":
        return 0.0
    if recipe == "fp8_current":
        return 2.0 + 3.0
    if recipe == "fp8_delayed":
        return 3.0
    if recipe in ("fp8_block128", "fp8_block128_pow2"):
        return 3.0 + (4.0 / 16384 if w2d else 4.0 / 128)
    if recipe == "fp8_block128_1d1d":
        return 3.0 + 4.0 / 128
    if recipe == "fp8_block128_2d2d":
        return 3.0 + 4.0 / 16384
    if recipe == "mxfp8":
        return 3.0 + 1.0 / 32
    if recipe == "mxfp4":
        return 2.5 + 1.0 / 32
    if recipe == "nvfp4":
        return 2.0 + 2.5 + (1.0 / 256 if w2d else 1.0 / 16)
    if recipe == "fp8_channel":
        return 3.0 + 4.0 / k_len
    raise ValueError(recipe)


def autocast_roofline_ms(runner, recipe, peak=None):
    """Per layer: GEMM flops at the recipe's matrix peak plus quantization
    bytes at 8 TB/s, both operands of every GEMM quantized (autocast)."""
    from precision_block_scaled_amd import pipeline as PL
    peak = peak or RECIPE_PEAK.get(recipe, 5033.2)
    t = 0.0
    for (_, p, M, N, K) in runner.gemms:
        t += 2.0 * M * N * K / (peak * 1e12)
        (sa, _), (sb, _) = PL.ROLES[p]
        q = M * K * quant_bytes_per_element(recipe, sa, K) + N * K * quant_bytes_per_element(recipe, sb, K)
        t += q / (HBM_GBPS * 1e9)
    return t * 1e3


def layer_roofline_ms(runner, recipe):
    """Per layer in layer-autocast mode: GEMM flops at the recipe's matrix
    peak plus one read of X, W and dY and the writes of both copies of each
    (the 4-bit recipes read X and dY once more for the Hadamard copy and its
    maximum; the maxima of X and dY come from the producers' epilogues)."""
    peak = RECIPE_PEAK.get(recipe, 5033.2)
    t = sum(2.0 * M * N * K for (_, _, M, N, K) in runner.gemms) / (peak * 1e12)
    if recipe == "bf16":
        return t * 1e3
    out_b = {"fp8_current": 1.0, "fp8_delayed": 1.0, "fp8_block128": 1.0 + 4 / 128, "mxfp8": 1.0 + 1 / 32,
             "nvfp4": 0.5 + 1 / 16, "mxfp4": 0.5 + 1 / 32, "fp8_channel": 1.0, "fp8_block128_pow2": 1.0 + 4 / 128,
             "fp8_block128_1d1d": 1.0 + 4 / 128, "fp8_block128_2d2d": 1.0}[recipe]
    q = 0.0
    for (x, w, dy, ls) in runner.layers.values():
        for t_, src in ((x, "x"), (w, "w"), (dy, "dy")):
            n = t_.numel()
            reads = 2.0
            if recipe in ("nvfp4", "mxfp4") and src != "w":
                reads = 2.0 * (3 if recipe == "nvfp4" else 2)     # row cast, RHT amax (NVFP4), RHT col cast
            if recipe == "fp8_current" and src == "w":
                reads = 4.0                                        # amax pass, then the cast
            if recipe == "nvfp4" and src == "w":
                reads = 4.0
            q += n * (reads + 2 * out_b)
    return (t + q / (HBM_GBPS * 1e9)) * 1e3


def recipe_table(runner, recipes, per, pre, cold=None, layer=None):
    """ms per layer and TFLOP/s per recipe: autocast (median and min over the
    timed steps), pre-quantized (median and min, operands hot in the caches;
    and with the caches flushed when `cold` is given), layer autocast; the
    fraction of each mode's roofline (for NVFP4 against the fp16 matrix
    rate it runs on and against the FP4 format's peak)."""
    out = {}
    layer_flop = sum(2.0 * M * N * K for (_, _, M, N, K) in runner.gemms)
    tf = lambda ms: round(layer_flop / (ms * 1e-3) / 1e12, 1)
    for r in recipes:
        auto_ms = sum(float(np.median(per[(r, n, p)]["auto"])) for (n, p, *_) in runner.gemms)
        auto_min = sum(float(np.min(per[(r, n, p)]["auto"])) for (n, p, *_) in runner.gemms)
        roof = autocast_roofline_ms(runner, r)
        ent = {"autocast_ms_per_layer": round(auto_ms, 3), "autocast_min_ms_per_layer": round(auto_min, 3),
               "autocast_TFLOPs": tf(auto_ms),
               "autocast_roofline_ms_per_layer": round(roof, 3),
               "autocast_roofline_frac": round(roof / auto_ms, 4)}
        if r in FORMAT_PEAK:
            roof_f = autocast_roofline_ms(runner, r, peak=FORMAT_PEAK[r])
            ent["autocast_roofline_frac_format_peak"] = round(roof_f / auto_ms, 4)
        if pre:
            pre_ms = sum(pre[(r, n, p)][0] for (n, p, *_) in runner.gemms)
            pre_min = sum(pre[(r, n, p)][1] for (n, p, *_) in runner.gemms)
            peak = RECIPE_PEAK.get(r, 5033.2)
            ent["prequant_ms_per_layer"] = round(pre_ms, 3)
            ent["prequant_min_ms_per_layer"] = round(pre_min, 3)
            ent["prequant_TFLOPs"] = tf(pre_ms)
            ent["prequant_frac_of_peak"] = round(layer_flop / (pre_ms * 1e-3) / 1e12 / peak, 4)
            if r in FORMAT_PEAK:
                ent["prequant_frac_of_format_peak"] = round(layer_flop / (pre_ms * 1e-3) / 1e12 / FORMAT_PEAK[r], 4)
            ent["ms_per_gemm_prequant"] = {f"{n}.{p}": round(pre[(r, n, p)][0], 4) for (n, p, *_) in runner.gemms}
            ent["ms_per_gemm_prequant_min"] = {f"{n}.{p}": round(pre[(r, n, p)][1], 4) for (n, p, *_) in runner.gemms}
        if cold:
            cold_ms = sum(cold[(r, n, p)][0] for (n, p, *_) in runner.gemms)
            ent["prequant_cold_ms_per_layer"] = round(cold_ms, 3)
            ent["prequant_cold_TFLOPs"] = tf(cold_ms)
        if layer and r in layer:
            ent["layer_autocast_ms_per_layer"] = round(layer[r], 3)
            ent["layer_autocast_TFLOPs"] = tf(layer[r])
            lroof = layer_roofline_ms(runner, r)
            ent["layer_autocast_roofline_ms_per_layer"] = round(lroof, 3)
            ent["layer_autocast_roofline_frac"] = round(lroof / layer[r], 4)
        out[r] = ent
    return out


def model_analysis(runner, recipes, per, pre, layers=24):
    """The pages' model-level reading of the per-GEMM times ("How to optimize
    Transformer-based models for low-precision training", "Using autocast mode
    vs pre-quantized mode" and "Interpreting results for a real model"):
    per-recipe speedup over BF16 in both modes, the model's GEMM time for its
    `layers` identical layers, the MXFP8 / NVFP4 Fprop ratio per layer, the Dgrad /
    Fprop asymmetry per layer, and the weight bytes each recipe stores."""
    P = runner.P
    names = [ls.name for (_, _, _, ls) in runner.layers.values()]
    med = lambda r, n, p: float(np.median(per[(r, n, p)]["auto"]))
    auto = {r: sum(med(r, n, p) for (n, p, *_) in runner.gemms) for r in recipes}
    out = {"layers": layers, "per_recipe": {}}
    for r in recipes:
        e = {"autocast_ms_per_model": round(layers * auto[r], 2)}
        if "bf16" in auto:
            e["speedup_vs_bf16_autocast"] = round(auto["bf16"] / auto[r], 3)
        if pre:
            pm = sum(pre[(r, n, p)][0] for (n, p, *_) in runner.gemms)
            e["prequant_ms_per_model"] = round(layers * pm, 2)
            if "bf16" in recipes:
                pb = sum(pre[("bf16", n, p)][0] for (n, p, *_) in runner.gemms)
                e["speedup_vs_bf16_prequant"] = round(pb / pm, 3)
        # stored weight bytes of the layer (codes + block scales + fp32 tensor scalars)
        wb = 0
        for (_, w, _, ls) in runner.layers.values():
            if r == "bf16":
                wb += w.numel() * 2
                continue
            rec = runner.PL.RECIPES[r]
            w2d = "w" in runner.PL.TWO_D.get(r, ())
            cb, sb = P.pbs_quantized_bytes(rec, ls.n_out, ls.k_in, int(w2d))
            wb += cb + sb + (4 if r in ("fp8_current", "fp8_delayed", "nvfp4") else 0)
        e["weight_MB_per_layer"] = round(wb / 1e6, 2)
        out["per_recipe"][r] = e
    if "mxfp8" in recipes and "nvfp4" in recipes:
        out["mxfp8_over_nvfp4_fprop_autocast"] = {n: round(med("mxfp8", n, "fprop") / med("nvfp4", n, "fprop"), 3)
                                                  for n in names}
    if pre:
        out["dgrad_over_fprop_prequant"] = {r: {n: round(pre[(r, n, "dgrad")][0] / pre[(r, n, "fprop")][0], 3) for n in names}
                                            for r in recipes}
    return out


def speedup_table(runner, recipes, per, pre=None):
    """Per GEMM of the layer, in runner.gemms order: {recipe: [value, ...]},
    the speedup over BF16 in the timed mode (autocast median, or
    pre-quantized when `pre` is given) when BF16 was run (BF16 itself then
    left out), else TFLOP/s.  Returns (labels, table, "speedup" | "TFLOP/s")."""
    ms = (lambda r, n, p: pre[(r, n, p)][0]) if pre else (lambda r, n, p: float(np.median(per[(r, n, p)]["auto"])))
    labels = [f"{n}.{p}" for (n, p, *_) in runner.gemms]
    if "bf16" in recipes:
        tab = {r: [ms("bf16", n, p) / ms(r, n, p) for (n, p, *_) in runner.gemms] for r in recipes if r != "bf16"}
        return labels, tab, "speedup"
    tab = {r: [2.0 * M * N * K / (ms(r, n, p) * 1e-3) / 1e12 for (n, p, M, N, K) in runner.gemms] for r in recipes}
    return labels, tab, "TFLOP/s"


def write_speedup_plot(path, runner, recipes, per, pre, title):
    """The chart the pages' benchmark writes with -o ("How to optimize
    Transformer-based models for low-precision training", "Model
    configuration and training inputs"): for each of the layer's GEMMs
    (Fprop, Dgrad, Wgrad of QKV, attention-out, MLP-up, MLP-down) one bar per
    recipe, from speedup_table.  Returns the path written."""
    import matplotlib
    matplotlib.use("Agg")
    import matplotlib.pyplot as plt
    labels, tab, kind = speedup_table(runner, recipes, per, pre)
    n = max(1, len(tab))
    fig, ax = plt.subplots(figsize=(max(8.0, 0.3 * len(labels) * n), 4.8))
    width = 0.8 / n
    xs = np.arange(len(labels))
    for i, (r, ys) in enumerate(tab.items()):
        ax.bar(xs + (i - (n - 1) / 2) * width, ys, width, label=r)
    if kind == "speedup":
        ax.axhline(1.0, color="black", linewidth=0.8)
    ax.set_xticks(xs)
    ax.set_xticklabels([l.replace(".", "\n") for l in labels], fontsize=7)
    ax.set_ylabel("speedup over BF16" if kind == "speedup" else "TFLOP/s")
    ax.set_title(title, fontsize=9)
    ax.legend(fontsize=7, ncol=min(n, 6))
    fig.tight_layout()
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    fig.savefig(path, dpi=120)
    plt.close(fig)
    return path


def host_info():
    """Host CPU facts for the oracle baseline."""
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        import threadpoolctl
        blas = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()), default=None)
    except Exception:
        pass
    return {"cpu_count": os.cpu_count(), "affinity_cores": cores, "cpu_model": model, "blas_threads": blas}


def _threads():
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return max(1, min(16, os.cpu_count() or 1))


def cpu_baseline(runner, per, pre, quant_gbps, seconds_target=8.0):
    """The CPU oracle beside the GPU, on bounded samples of the same workload.

    * value: autocast Fprop of the attention-out layer (W [4096, 4096]) for
      256 tokens, all six recipes (oracle quantize of X and W, then the fp64
      GEMM over the dequantized operands), repeated for about
      `seconds_target` seconds: TFLOP/s of the oracle doing what a step does;
    * per recipe, the oracle's quantization of a [512, 16384] slice of the
      MLP-down activations (row chunks over the host's threads): GB/s in the
      same algorithmic bytes as the GPU's quantize passes, and the GPU/CPU
      ratio where the GPU timed the same cast;
    * the fp64 GEMM of each of the 12 GEMMs on a 256-row slice (full K and
      N), extrapolated to the full M, beside the GPU's per-GEMM autocast
      time of each recipe; one full-shape fp64 GEMM (MLP-down Fprop)
      calibrates the extrapolation."""
    import concurrent.futures as cf
    import workloads as W
    from oracle import recipes as R
    from oracle.passes import pass_operands
    from oracle.gemm_ref import gemm_ref
    info = host_info()
    nthr = _threads()
    rows = 256
    x = W.activations(rows, 4096, seed=11)
    w = W.weights(4096, 4096, seed=21)
    dy = W.grads(rows, 4096, seed=31)
    flop = 0.0
    passes = 0
    t0 = time.perf_counter()
    while passes == 0 or time.perf_counter() - t0 < seconds_target:
        for r in RECIPES:
            st = None
            if r == "fp8_delayed":
                st = {"x": R.DelayedScaling("e4m3"), "w": R.DelayedScaling("e4m3")}
                st["x"].update(R.amax(x))
                st["w"].update(R.amax(w))
            A, B = pass_operands(r, "fprop", x=x, w=w, dy=dy, delayed_states=st)
            gemm_ref(A.dequant(), B.dequant())
            flop += 2.0 * rows * 4096 * 4096
        passes += 1
    dt = time.perf_counter() - t0

    # quantization of a [512, 16384] activation slice, row chunks in threads
    xq = W.activations(512, 16384, seed=13)
    chunks = np.array_split(np.arange(512), nthr)
    quant = {}
    label = {"fp8_current": "fp8_tensor_cast_row", "fp8_block128": "fp8_block128_cast_row",
             "mxfp8": "mxfp8_cast_row", "nvfp4": "nvfp4_cast_row"}
    from oracle.formats import bf16_to_f32
    S_nv = R.nvfp4_tensor_scales(R.amax(xq))[0]
    s_cur = R.scale_from_amax(R.amax(xq), 448.0)[0]
    casts = {"fp8_current": lambda c: R.cast_pertensor(xq[c], s_cur, "e4m3", "row"),
             "fp8_block128": lambda c: R.quantize_block128(xq[c], "row"),
             "mxfp8": lambda c: R.quantize_mxfp8(xq[c], "row"),
             "nvfp4": lambda c: R.quantize_nvfp4(bf16_to_f32(xq[c]), S_nv)}
    for r, fn in casts.items():
        tq = time.perf_counter()
        with cf.ThreadPoolExecutor(nthr) as ex:
            list(ex.map(fn, chunks))
        tq = time.perf_counter() - tq
        # the cast's own bytes (without the amax pass), as the GPU's GB/s counts them
        bpe = quant_bytes_per_element(r, "x", 16384) - (2.0 if r in ("fp8_current", "nvfp4") else 0.0)
        gbps = bpe * xq.size / tq / 1e9
        e = {"ms": round(tq * 1e3, 2), "GBps": round(gbps, 3), "elements": int(xq.size), "threads": nthr}
        g = quant_gbps.get(label[r], {}).get("GBps") if quant_gbps else None
        if g:
            e["gpu_GBps"] = g
            e["gpu_over_cpu"] = round(g / gbps, 1)
        quant[r] = e

    # fp64 GEMMs: 256-row slices of the 12 GEMMs, extrapolated to the full M
    rng = np.random.default_rng(0)
    gemms = {}
    t_oracle_layer = 0.0
    for (name, p, M, N, K) in runner.gemms:
        a = rng.standard_normal((256, K))
        b = rng.standard_normal((N, K))
        tg = time.perf_counter()
        a @ b.T
        tg = time.perf_counter() - tg
        ext = tg * M / 256 * 1e3
        t_oracle_layer += ext
        gemms[f"{name}.{p}"] = {"oracle_fp64_ms_extrapolated": round(ext, 1)}
    gpu_layer = {r: sum(float(np.median(per[(r, n, p)]["auto"])) for (n, p, *_) in runner.gemms)
                 for r in RECIPES if (r, runner.gemms[0][0], runner.gemms[0][1]) in per}
    for (name, p, M, N, K) in runner.gemms:
        gemms[f"{name}.{p}"]["gpu_autocast_ms"] = {r: round(float(np.median(per[(r, name, p)]["auto"])), 4)
                                                   for r in gpu_layer}
    # one full-shape calibration: MLP-down Fprop
    calib = None
    md = next((g for g in runner.gemms if g[0] == "mlp_down" and g[1] == "fprop"), None)
    if md is not None:
        _, _, M, N, K = md
        a = rng.standard_normal((M, K))
        b = rng.standard_normal((N, K))
        tg = time.perf_counter()
        a @ b.T
        tg = time.perf_counter() - tg
        del a, b
        calib = {"gemm": f"mlp_down.fprop [{M}x{K}]x[{K}x{N}] fp64, full shape", "ms": round(tg * 1e3, 1),
                 "extrapolated_from_256_rows_ms": gemms["mlp_down.fprop"]["oracle_fp64_ms_extrapolated"]}
    layer_flop = sum(2.0 * M * N * K for (_, _, M, N, K) in runner.gemms)
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": info["blas_threads"] or info["affinity_cores"],
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"autocast Fprop of attn-out (W 4096x4096) for {rows} tokens, all 6 recipes: "
                      f"oracle quantize of X and W + fp64 GEMM, {passes} passes",
            "host": info,
            "quantize_512x16384_activations": quant,
            "fp64_gemm_per_layer_ms_extrapolated": round(t_oracle_layer, 1),
            "fp64_gemm_TFLOPs": round(layer_flop / (t_oracle_layer * 1e-3) / 1e12, 3),
            "gpu_autocast_ms_per_layer": {r: round(v, 3) for r, v in gpu_layer.items()},
            "gpu_over_cpu_per_layer": {r: round(t_oracle_layer / v, 1) for r, v in gpu_layer.items()},
            "per_gemm": gemms, "calibration": calib}


def fp8_exceedance(runner, recipes, group_rows=128):
    """How far the FP8-instruction GEMMs land outside the stated tolerance
    alone, 1e-5 * sum|a b| + one bf16 ulp (the oracle accepts them with the
    8-bit dot unit's term added): the Fprop GEMM of every layer, its outputs
    at one 128-row group of X x one 128-row group of W (the middle ones),
    against the oracle's fp64 product of those rows quantized on the host."""
    import workloads as W
    from oracle import recipes as R
    from oracle.gemm_ref import check_gemm, fp8_dot_unit_bound
    from oracle.passes import quantize_operand
    torch, PL = runner.torch, runner.PL
    out = {}
    for r in recipes:
        if r in ("bf16", "nvfp4", "mxfp4"):
            continue
        worst, over, total, outside = 0.0, 0, 0, 0
        for (name, p, M, N, K) in runner.gemms:
            if p != "fprop" or (r, name, p) not in runner.q:
                continue
            x, w, dy, ls = runner.layers[name]
            A, B = runner.q[(r, name, p)]
            C = PL.gemm(r, p, A, B, M, N, K)
            ra = np.arange(group_rows) + (M // group_rows // 2) * group_rows
            rb = np.arange(group_rows) + (N // group_rows // 2) * group_rows
            c = C[torch.from_numpy(ra).to(C.device)][:, torch.from_numpy(rb).to(C.device)].float().cpu().numpy()
            xb = x.view(torch.int16).cpu().numpy().view(np.uint16)
            wb = w.view(torch.int16).cpu().numpy().view(np.uint16)
            if r in ("fp8_current", "fp8_delayed"):
                sa = R.scale_from_amax(R.amax(xb), 448.0)
                sb = R.scale_from_amax(R.amax(wb), 448.0)
                ah = R.dequant_pertensor(R.cast_pertensor(xb[ra], sa[0], "e4m3"), "e4m3", sa[1])
                bh = R.dequant_pertensor(R.cast_pertensor(wb[rb], sb[0], "e4m3"), "e4m3", sb[1])
            else:
                ah = quantize_operand(r, "x", "row", xb[ra], "fprop").dequant()
                bh = quantize_operand(r, "w", "row", wb[rb], "fprop").dequant()
            cref = ah @ bh.T
            base = np.abs(ah) @ np.abs(bh).T
            ok0, tol0, err = check_gemm(c, cref, base, True)      # 1e-5 sum|ab| + 1 bf16 ulp
            worst = max(worst, float((err / tol0).max()))
            over += int((~ok0).sum())
            outside += int((~check_gemm(c, cref, base, True, fp8_dot_unit_bound(ah, bh))[0]).sum())
            total += c.size
        out[r] = {"outputs": total, "max_err_over_stated_bound": round(worst, 3),
                  "outputs_over_stated_bound": over, "outputs_outside_oracle_tolerance": outside}
    return out


def load_traffic(kernel_name):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except Exception:
        return None
    rec = d.get(kernel_name)
    if not rec or rec.get("source_digest") != source_digest(kernel_source_files(kernel_name)):
        return None
    return rec


def timed_steps(runner, recipes, warmup, steps, prequant_mode):
    """Warm-up, then `steps` timed steps bracketed by device synchronisation.
    Returns (wall ms per step, events).  In pre-quantized mode the operands
    are quantized once by the warm-up and each step runs the GEMMs only."""
    torch = runner.torch
    for _ in range(max(1, warmup) if prequant_mode else warmup):
        runner.step(recipes)
    torch.cuda.synchronize()
    events = []
    t0 = time.perf_counter()
    for _ in range(steps):
        if prequant_mode:
            runner.gemm_step(recipes, events)
        else:
            runner.step(recipes, events)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps, events


def layer_mode(runner, recipes, warmup, steps):
    """ms per layer of the layer-autocast mode, per recipe (median of steps)."""
    torch = runner.torch
    runner.prepare_layer_mode()
    for _ in range(warmup):
        runner.layer_step(recipes, [])
    ev = []
    for _ in range(steps):
        runner.layer_step(recipes, ev)
    torch.cuda.synchronize()
    acc = {}
    for (r, name, e0, e1) in ev:
        acc.setdefault(r, {}).setdefault(name, []).append(e0.elapsed_time(e1))
    return {r: sum(float(np.median(v)) for v in d.values()) for r, d in acc.items()}


def sweep(cfg, tokens, recipes, dev, warmup, steps, iters):
    """The six recipes on another configuration (autocast and pre-quantized
    ms per layer, TFLOP/s and roofline fractions), reported apart from value."""
    torch = __import__("torch")
    layers = build_layer_tensors(cfg, tokens, dev)
    runner = Runner(layers, tokens, dev)
    ms_step, events = timed_steps(runner, recipes, warmup, steps, False)
    per, _ = per_gemm_times(events)
    pre = runner.prequant_pass(recipes, iters)
    tab = recipe_table(runner, recipes, per, pre)
    for r in tab:
        tab[r].pop("ms_per_gemm_prequant_min", None)
    out = {"tokens": tokens, **{k: cfg[k] for k in ("hidden", "intermediate", "heads", "kv_heads", "gated")},
           "gemm_shapes_MNK": {f"{n}.{p}": [M, N, K] for (n, p, M, N, K) in runner.gemms},
           "layer_TFLOP": round(sum(2.0 * M * N * K for (_, _, M, N, K) in runner.gemms) / 1e12, 3),
           "ms_per_step": round(ms_step, 3), "per_recipe": tab}
    del runner, layers
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    # model configuration and batch, as the pages' benchmark takes them
    ap.add_argument("--model", choices=sorted(MODELS), default="codonfm",
                    help="preset the flags below are defaults of")
    ap.add_argument("--hidden_size", "--hidden-size", type=int, default=None)
    ap.add_argument("--intermediate_size", "--intermediate-size", type=int, default=None)
    ap.add_argument("--num_attention_heads", "--num-attention-heads", type=int, default=None)
    ap.add_argument("--num_key_value_heads", "--num-key-value-heads", type=int, default=None)
    ap.add_argument("--num_hidden_layers", "--num-hidden-layers", type=int, default=None,
                    help="layers of the model-level projection (identical layers)")
    ap.add_argument("--gated", choices=("yes", "no"), default=None, help="gated MLP (up projection 2x wide)")
    ap.add_argument("--micro_batch_size", "--micro-batch-size", type=int, default=None)
    ap.add_argument("--sequence_length", "--sequence-length", type=int, default=None)
    ap.add_argument("--tokens", type=int, default=None, help="tokens per step (overrides micro-batch x sequence)")
    ap.add_argument("--pre-quantize", "--pre_quantize", action="store_true",
                    help="time the GEMMs alone on operands quantized before the timed steps")
    ap.add_argument("--recipes", default=",".join(RECIPES))
    ap.add_argument("--no-fp8", "--no_fp8", action="store_true", help="drop MXFP8 from the recipes")
    ap.add_argument("--no-fp4", "--no_fp4", action="store_true",
                    help="drop the 4-bit recipes (NVFP4, and MXFP4 of the next recipes)")
    ap.add_argument("-o", "--output", default=None,
                    help="write the per-GEMM speedup-over-BF16 chart of the timed mode to this image file")
    ap.add_argument("--next-recipes", default=",".join(NEXT_RECIPES),
                    help="recipes beyond the six, timed after the step and reported apart")
    ap.add_argument("--prequant-iters", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip every pass after the timed steps")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the 32768-token CodonFM and 8192-token Llama-3-8B sweeps")
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run a plain device copy of known size (counter calibration)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {a.gpus}); the multi-GPU "
              "sharding of this path is a design note, not built.", file=sys.stderr)
        sys.exit(2)
    cfg = dict(MODELS[a.model])
    for key, val in (("hidden", a.hidden_size), ("intermediate", a.intermediate_size),
                     ("heads", a.num_attention_heads), ("kv_heads", a.num_key_value_heads),
                     ("micro_batch", a.micro_batch_size), ("seq_len", a.sequence_length),
                     ("num_layers", a.num_hidden_layers)):
        if val is not None:
            cfg[key] = val
    if a.num_attention_heads is not None and a.num_key_value_heads is None and a.model == "codonfm":
        cfg["kv_heads"] = cfg["heads"]
    if a.gated is not None:
        cfg["gated"] = a.gated == "yes"
    tokens = a.tokens if a.tokens is not None else cfg["micro_batch"] * cfg["seq_len"]

    import torch
    dev = torch.device("cuda:0")
    if a.calib_copy:
        n = 1 << 28                       # 256 Mi float32 = 1 GiB each way
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes_each_way": n * 4}))
        return

    import precision_block_scaled_amd as P
    P.lib()
    dropped = ({"mxfp8"} if a.no_fp8 else set()) | ({"nvfp4", "mxfp4"} if a.no_fp4 else set())
    recipes = [r for r in a.recipes.split(",") if r and r not in dropped]
    log(f"generating inputs: {a.model} {cfg} tokens={tokens}")
    layers = build_layer_tensors(cfg, tokens, dev)
    runner = Runner(layers, tokens, dev)
    total_flop = sum(2.0 * M * N * K for (_, _, M, N, K) in runner.gemms) * len(recipes)

    clock = ClockSampler()      # shader clock over the GEMM-heavy part (warm-up to pre-quantized)
    clock.__enter__()
    log(f"warmup {a.warmup}, timing {a.steps} steps ({'pre-quantized' if a.pre_quantize else 'autocast'})")
    ms_step, events = timed_steps(runner, recipes, a.warmup, a.steps, a.pre_quantize)

    per, kern = per_gemm_times(events)
    dom = max(kern.items(), key=lambda kv: kv[1]["ms"])
    dom_name, dk = dom
    avg_ms = dk["ms"] / dk["launches"]
    achieved = dk["flop"] / (dk["ms"] * 1e-3) / 1e12
    peak = PEAK_TFLOPS[dk["dtype"]]
    traffic = load_traffic(dom_name)

    pre, cold, lay = {}, {}, {}
    if not a.no_extras:
        if a.pre_quantize:          # the timed steps were the GEMMs alone: fill the autocast table too
            ev_a = []
            for _ in range(a.steps):
                runner.step(recipes, ev_a)
            torch.cuda.synchronize()
            per, _ = per_gemm_times(ev_a)
        log("pre-quantized GEMM timing (operands hot, then with the caches flushed)")
        pre = runner.prequant_pass(recipes, a.prequant_iters)
        cold = runner.prequant_pass(recipes, a.prequant_iters, cold=True)
        log("layer autocast (each tensor quantized once per layer)")
        lay = layer_mode(runner, recipes, a.warmup, a.steps)
    clock.__exit__(None, None, None)
    per_recipe = recipe_table(runner, recipes, per, pre, cold, lay)
    epi = epilogue_amax_cost(runner) if (not a.no_extras and "fp8_current" in recipes) else None
    model = model_analysis(runner, recipes, per, pre, layers=cfg["num_layers"])
    plot_path = None
    if a.output:
        mode = "pre-quantized" if a.pre_quantize else "autocast"
        if a.pre_quantize and not pre:
            log("-o: the pre-quantized chart needs the pre-quantized pass (not run with --no-extras)")
        else:
            plot_path = write_speedup_plot(
                a.output, runner, recipes, per, pre if a.pre_quantize else None,
                f"{a.model}: hidden {cfg['hidden']}, intermediate {cfg['intermediate']}, {tokens} tokens, {mode}")
            log(f"wrote {plot_path}")

    next_recipes = [r for r in a.next_recipes.split(",") if r and r not in dropped]
    nxt = {}
    if not a.no_extras and next_recipes:
        log(f"next recipes {next_recipes} (reported apart from value)")
        _, ev2 = timed_steps(runner, next_recipes, a.warmup, a.steps, False)
        per2, kern2 = per_gemm_times(ev2)
        pre2 = runner.prequant_pass(next_recipes, a.prequant_iters)
        lay2 = layer_mode(runner, next_recipes, a.warmup, a.steps)
        nxt = recipe_table(runner, next_recipes, per2, pre2, None, lay2)
        for key, k in kern2.items():
            tf = k["flop"] / (k["ms"] * 1e-3) / 1e12
            nxt.setdefault("kernels", {})[key] = {
                "avg_launch_ms": round(k["ms"] / k["launches"], 4), "achieved_TFLOPs": round(tf, 1),
                "peak": PEAK_TFLOPS[k["dtype"]], "frac": round(tf / PEAK_TFLOPS[k["dtype"]], 4)}
    qbw = {}
    exceed = None
    if not a.no_extras:
        log("quantize-pass bandwidth")
        qbw = quant_bandwidth(runner)
        if not a.no_cpu_baseline:
            log("FP8-instruction outputs against the stated tolerance (oracle on sampled rows)")
            exceed = fp8_exceedance(runner, recipes + [r for r in next_recipes if r not in recipes])

    cpu = None
    if not a.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(runner, per, pre, qbw)

    sweeps = {}
    if not a.no_extras and not a.no_sweep:
        del runner, layers
        torch.cuda.empty_cache()
        for label, mname, tok in (("codonfm_32768_tokens", "codonfm", 32768), ("llama3_8b_8192_tokens", "llama3_8b", 8192)):
            log(f"sweep {label}")
            sweeps[label] = sweep(MODELS[mname], tok, recipes, dev, 1, max(2, a.steps // 2), max(2, a.prequant_iters // 2))

    roof = {"kernel": dom_name, "bound": "mfma", "achieved": round(achieved, 1),
            "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
            "avg_launch_ms": round(avg_ms, 4), "launches": dk["launches"],
            # HBM bytes per launch from the committed rocprofv3 counters (null once
            # the kernel's sources differ from those the counters were taken on)
            "traffic": round(traffic["bytes_per_launch"]) if traffic else None,
            "traffic_fetch_write": ([round(traffic["fetch_bytes_per_launch"]),
                                     round(traffic["write_bytes_per_launch"])] if traffic else None)}
    if dom_name.startswith("gemm_nvfp4"):       # the 4-bit format's own peak, beside the fp16 instruction's
        roof["format_peak_fp4"] = PEAK_TFLOPS["fp4"]
        roof["frac_of_format_peak_fp4"] = round(achieved / PEAK_TFLOPS["fp4"], 4)
    same_layer = all(cfg[k] == MODELS["codonfm"][k] for k in ("hidden", "intermediate", "heads", "kv_heads", "gated"))
    layer_desc = ("CodonFM-5B layer" if a.model == "codonfm" and same_layer else
                  f"{a.model}-shaped layer (hidden {cfg['hidden']}, intermediate {cfg['intermediate']}, "
                  f"heads {cfg['heads']}/{cfg['kv_heads']} kv, gated {cfg['gated']})")
    line = {
        "metric": "TFLOPS & ms/GEMM over 12 layer shapes (M=15872) per recipe; quant GB/s",
        "value": round(total_flop / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mixed: bf16 | fp8 (e4m3/e5m2) | nvfp4 decoded to fp16",
        "data": "synthetic (seeded N(0,1)+8 outlier channels x100, N(0,0.02^2), Student-t(3)x1e-3)",
        "config": {"workload": f"{layer_desc}, 12 GEMMs (QKV/attn-out/MLP-up/MLP-down x Fprop/Dgrad/Wgrad), "
                               f"{'pre-quantized' if a.pre_quantize else 'autocast'}, every recipe",
                   "tokens": tokens, "hidden": cfg["hidden"], "intermediate": cfg["intermediate"],
                   "heads": cfg["heads"], "kv_heads": cfg["kv_heads"], "gated": cfg["gated"],
                   "micro_batch": cfg["micro_batch"], "seq_len": cfg["seq_len"],
                   "mode": "pre-quantized" if a.pre_quantize else "autocast",
                   "recipes": recipes, "gemm_out": "bf16", "parallelism": "single GPU"},
        "roofline": roof,
        "per_recipe": per_recipe,
        "next_recipes": nxt,
        "model": model,
        "sweep": sweeps,
        "quant_GBps": qbw,
        "epilogue_amax": epi,
        "fp8_tolerance_exceedance": exceed,
        "gpu_clock": clock.summary(),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
