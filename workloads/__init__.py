"""Seeded synthetic inputs and the GEMM shapes of a Transformer layer.

This module is shared by the CPU oracle and the HIP path as the single
source of their inputs; it holds none of the quantization arithmetic.

Shapes ("How to optimize Transformer-based models for low-precision
training", "Model configuration and training inputs" and "Using autocast
mode vs pre-quantized mode"): a model configuration and a batch become the
exact M x K x N problems of the linear layers.  With M = micro_batch *
sequence tokens, each layer runs four linear layers (QKV projection,
attention output, MLP up, MLP down), each in three passes (Fprop, Dgrad,
Wgrad): twelve GEMMs, benchmarked separately because the aspect ratio
changes between the passes.

Distributions (the recipe every test and the benchmark use):
  * activations X [M, K]: N(0, 1), with 8 outlier channels (columns chosen
    without replacement) multiplied by 100;
  * weights W, stored [N, K] (Linear convention): N(0, 0.02**2);
  * output gradients dY [M, N]: Student-t with 3 degrees of freedom, * 1e-3;
  * the tiny per-tensor case: A [256, 512] N(0,1) with a Bernoulli(0.01)
    mask of entries multiplied by 50, B [512, 256] N(0, 0.02**2), seed 0.
fp32 draws become bf16 by round-to-nearest-even.  Large tensors are drawn in
row chunks, each from its own child of one ``SeedSequence``, so the bytes do
not depend on the number of threads used to draw them.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass

import numpy as np

# ---------------------------------------------------------------------------
# shapes
# ---------------------------------------------------------------------------
PASSES = ("fprop", "dgrad", "wgrad")
LAYERS = ("qkv", "attn_out", "mlp_up", "mlp_down")


@dataclass(frozen=True)
class LayerShape:
    name: str
    k_in: int      # input features (contraction dim of Fprop)
    n_out: int     # output features


@dataclass(frozen=True)
class GemmShape:
    layer: str
    pass_: str
    m: int         # rows of the output
    k: int         # contraction length
    n: int         # columns of the output

    @property
    def flop(self):
        return 2 * self.m * self.k * self.n


def layer_shapes(hidden, intermediate, heads, kv_heads=None, gated=False):
    kv_heads = heads if kv_heads is None else kv_heads
    head_dim = hidden // heads
    n_qkv = hidden + 2 * kv_heads * head_dim
    n_up = intermediate * (2 if gated else 1)
    return [LayerShape("qkv", hidden, n_qkv),
            LayerShape("attn_out", hidden, hidden),
            LayerShape("mlp_up", hidden, n_up),
            LayerShape("mlp_down", intermediate, hidden)]


def gemm_shapes(hidden, intermediate, heads, micro_batch, seq_len, kv_heads=None,
                gated=False, tokens=None):
    """The 12 (layer, pass) GEMMs.  Fprop Y = X W^T: (M, K, N); Dgrad
    dX = dY W: (M, N, K); Wgrad dW = X^T dY: (K, M, N)."""
    m = micro_batch * seq_len if tokens is None else tokens
    out = []
    for ls in layer_shapes(hidden, intermediate, heads, kv_heads, gated):
        out.append(GemmShape(ls.name, "fprop", m, ls.k_in, ls.n_out))
        out.append(GemmShape(ls.name, "dgrad", m, ls.n_out, ls.k_in))
        out.append(GemmShape(ls.name, "wgrad", ls.k_in, m, ls.n_out))
    return out


CODONFM_5B = dict(hidden=4096, intermediate=16384, heads=32, layers=24,
                  micro_batch=31, seq_len=512)
LLAMA3_8B_LAYER = dict(hidden=4096, intermediate=14336, heads=32, kv_heads=8, gated=True,
                       micro_batch=1, seq_len=8192)


def codonfm_shapes(tokens=None):
    c = CODONFM_5B
    return gemm_shapes(c["hidden"], c["intermediate"], c["heads"], c["micro_batch"],
                       c["seq_len"], tokens=tokens)


# ---------------------------------------------------------------------------
# bf16 conversion of generated values (input preparation, not the method)
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(x):
    """float32 -> bf16 bit patterns (uint16), round-to-nearest-even, finite inputs."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# chunked, thread-count-independent generation
# ---------------------------------------------------------------------------
_CHUNK_ROWS = 256


def _workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _chunked_bf16(seed, rows, cols, draw):
    """bf16 [rows, cols]; rows split in chunks, chunk i drawn by draw(Generator, nrows, cols)."""
    out = np.empty((rows, cols), dtype=np.uint16)
    n_chunks = max(1, (rows + _CHUNK_ROWS - 1) // _CHUNK_ROWS)
    children = np.random.SeedSequence(seed).spawn(n_chunks)

    def work(i):
        r0 = i * _CHUNK_ROWS
        r1 = min(rows, r0 + _CHUNK_ROWS)
        g = np.random.Generator(np.random.PCG64(children[i]))
        out[r0:r1] = f32_to_bf16_bits(draw(g, r1 - r0, cols))

    if n_chunks == 1:
        work(0)
    else:
        with _cf.ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(work, range(n_chunks)))
    return out


def activations(rows, cols, seed=1, n_outlier_channels=8, outlier_scale=100.0):
    """X [rows, cols] bf16 bits: N(0,1) with outlier channels * outlier_scale."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0x0C4A])))
    chans = g.choice(cols, size=min(n_outlier_channels, cols), replace=False)
    mult = np.ones(cols, dtype=np.float32)
    mult[chans] = np.float32(outlier_scale)

    def draw(gen, r, c):
        return gen.standard_normal((r, c), dtype=np.float32) * mult
    return _chunked_bf16(seed, rows, cols, draw)


def weights(n_out, k_in, seed=2, std=0.02):
    """W [n_out, k_in] bf16 bits ~ N(0, std**2)."""
    def draw(gen, r, c):
        return gen.standard_normal((r, c), dtype=np.float32) * np.float32(std)
    return _chunked_bf16(seed, n_out, k_in, draw)


def grads(rows, cols, seed=3, dof=3.0, scale=1e-3):
    """dY [rows, cols] bf16 bits ~ Student-t(dof) * scale."""
    def draw(gen, r, c):
        return (gen.standard_t(dof, size=(r, c)) * scale).astype(np.float32)
    return _chunked_bf16(seed, rows, cols, draw)


def drift(x_bits, step, factor=1.1):
    """bf16(fp32(x) * fp32(factor**step)): the step-s tensor of a drifting amax."""
    f = np.float32(factor ** step)
    return f32_to_bf16_bits(bf16_bits_to_f32(x_bits) * f)


def drift_factor(step, factor=1.1):
    return np.float32(factor ** step)


def tiny_current_case(seed=0):
    """A [256, 512] N(0,1) with 1% of entries * 50; B [512, 256] N(0, 0.02**2).

    Draw order: A normal, mask uniform, B normal.  Returns (A bits [256, 512],
    B bits stored as W [256, 512] = B^T, i.e. contraction-contiguous).
    """
    g = np.random.Generator(np.random.PCG64(seed))
    a = g.standard_normal((256, 512), dtype=np.float32)
    mask = g.random((256, 512), dtype=np.float32) < np.float32(0.01)
    a = np.where(mask, a * np.float32(50.0), a).astype(np.float32)
    b = (g.standard_normal((512, 256), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    return f32_to_bf16_bits(a), f32_to_bf16_bits(np.ascontiguousarray(b.T))


def all_bf16_patterns(exclude_nonfinite=True):
    """Every bf16 bit pattern once, as a [256, 256] tensor (non-finite ones zeroed)."""
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
    if exclude_nonfinite:
        exp = (b >> 7) & 0xFF
        b = np.where(exp == 0xFF, np.uint16(0), b).astype(np.uint16)
    return b
