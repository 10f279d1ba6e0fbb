"""The oracle's operand roles, pinned against the three products of a linear
layer formed directly from X, W and dY ("How to optimize Transformer-based
models for low-precision training", "Using autocast mode vs pre-quantized
mode": Fprop, Dgrad and Wgrad are separate GEMMs; "Interpreting results for a
real model": Dgrad swaps the roles of K and N).

With X [M, K], W stored [N, K] and dY [M, N]:
  Fprop  Y  = X . W^T   [M, N]
  Dgrad  dX = dY . W    [M, K]
  Wgrad  dW = X^T . dY  [K, N]
For the BF16 recipe the dequantized operands are the tensors themselves, so
the oracle's product must equal these (up to fp64 summation order).  For
every quantized recipe it must approximate them to within the recipe's
quantization error, which a swapped or untransposed copy would not -- also
on a layer with N == K, where shapes cannot tell the copies apart.
"""
import numpy as np
import pytest

import workloads as W
from oracle.formats import bf16_to_f32
from oracle.gemm_ref import gemm_ref
from oracle.passes import ALL_RECIPES, pass_operands
from oracle import recipes as R


def _layer(M, K, N, seed):
    return W.activations(M, K, seed=seed), W.weights(N, K, seed=seed + 1), W.grads(M, N, seed=seed + 2)


def _exact(pass_, x, w, dy):
    X, Wt, D = (bf16_to_f32(t).astype(np.float64) for t in (x, w, dy))
    return {"fprop": X @ Wt.T, "dgrad": D @ Wt, "wgrad": X.T @ D}[pass_]


SHAPES = [(128, 256, 384), (128, 256, 256)]    # (M, K, N): non-square, and N == K


@pytest.mark.parametrize("M,K,N", SHAPES)
@pytest.mark.parametrize("pass_", ["fprop", "dgrad", "wgrad"])
def test_bf16_roles_are_the_layer_products(M, K, N, pass_):
    x, w, dy = _layer(M, K, N, 3)
    a, b = pass_operands("bf16", pass_, x=x, w=w, dy=dy)
    c, base = gemm_ref(a.dequant(), b.dequant())
    want = _exact(pass_, x, w, dy)
    assert c.shape == want.shape
    assert (np.abs(c - want) <= 1e-12 * base).all()
    # the wrong copy is caught on the square layer too
    if N == K and pass_ == "dgrad":
        wrong = bf16_to_f32(dy).astype(np.float64) @ bf16_to_f32(w).astype(np.float64).T
        assert not (np.abs(c - wrong) <= 1e-3 * base).all()


REL = {"nvfp4": 0.25, "mxfp4": 0.3}     # 4-bit values; every 8-bit recipe well under 0.1


@pytest.mark.parametrize("M,K,N", SHAPES)
@pytest.mark.parametrize("recipe", [r for r in ALL_RECIPES if r != "bf16"])
@pytest.mark.parametrize("pass_", ["fprop", "dgrad", "wgrad"])
def test_quantized_roles_approximate_the_layer_products(M, K, N, recipe, pass_):
    x, w, dy = _layer(M, K, N, 5)
    st = None
    if recipe == "fp8_delayed":
        st = {k: R.DelayedScaling("e5m2" if k == "dy" else "e4m3") for k in ("x", "w", "dy")}
        for k, t in (("x", x), ("w", w), ("dy", dy)):
            st[k].update(R.amax(t))
    a, b = pass_operands(recipe, pass_, x=x, w=w, dy=dy, delayed_states=st)
    c, _ = gemm_ref(a.dequant(), b.dequant())
    want = _exact(pass_, x, w, dy)
    assert c.shape == want.shape
    rel = np.linalg.norm(c - want) / np.linalg.norm(want)
    assert rel < REL.get(recipe, 0.1), rel
