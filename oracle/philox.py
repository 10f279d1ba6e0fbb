"""Philox4x32-10 counter-based generator.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel
Random Numbers: As Easy as 1, 2, 3", SC'11, section 3 (the Philox
S-box: two 32x32->64 multiplications per round, a Feistel-like permutation
of the four counter words, a Weyl key schedule), with N=4 words of W=32 bits
and R=10 rounds.  The stochastic rounding of gradients named in "How to
optimize Transformer-based models for low-precision training",
"Interpreting results for a real model", uses it with key (42, 0); element
i of the gradient takes word i % 4 of the call with counter i // 4 (the
plainest reading of a counter-based generator keyed by a seed that spends
every word it makes).

One round, for counter (c0, c1, c2, c3) and key (k0, k1):
  (hi0, lo0) = M0 * c0        (hi1, lo1) = M1 * c2      (64-bit products)
  counter'   = (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0)
and between rounds the key advances by the Weyl constants (W0, W1).
"""
from __future__ import annotations

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9        # golden ratio
W1 = 0xBB67AE85        # sqrt(3) - 1

_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10.  All inputs uint32-like; returns 4 uint32 arrays."""
    c0 = np.asarray(c0, dtype=np.uint64)
    c1 = np.asarray(c1, dtype=np.uint64)
    c2 = np.asarray(c2, dtype=np.uint64)
    c3 = np.asarray(c3, dtype=np.uint64)
    k0 = np.uint64(k0)
    k1 = np.uint64(k1)
    c0, c1, c2, c3 = np.broadcast_arrays(c0, c1, c2, c3)
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + np.uint64(W0)) & _MASK32
            k1 = (k1 + np.uint64(W1)) & _MASK32
        p0 = np.uint64(M0) * c0          # < 2**64: no wrap
        p1 = np.uint64(M1) * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0)
    return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))


def philox_word_for_index(idx, seed=42):
    """The stochastic-rounding word of element idx: word idx % 4 of
    Philox4x32-10(key=(seed lo, seed hi), counter=(q lo, q hi, 0, 0)), q = idx // 4.

    One call of the generator yields four 32-bit words; four consecutive
    indices share a call, so a stream of n words costs n / 4 calls.
    """
    idx = np.asarray(idx, dtype=np.uint64)
    q = idx >> np.uint64(2)
    k = (idx & np.uint64(3)).astype(np.int64)
    seed = int(seed)
    w = philox4x32_10(q & _MASK32, q >> np.uint64(32), 0, 0, seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    return np.choose(k, w).astype(np.uint32)
