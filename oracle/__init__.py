"""CPU oracle for block-scaled quantize-then-GEMM.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
restatement of what the quantize-then-GEMM path computes, written from the
pages' description of the recipes.  Only the test-suite, the smoke check and
the ``cpu_baseline`` leg of the benchmark may import it.  The HIP library and
its Python binding never import, link or call anything in here, and nothing
in here imports them: the two sides share no code, table or constant
generator.  The seeded input generators live in the separate ``workloads``
package, which holds none of the method's arithmetic.

Pages cited in this package (title, then the section used):

* "Optimizing Transformer models for low-precision training" (setupai digest
  of the NVIDIA blog post) -- "Technical deep-dive": the E4M3 / E5M2 bit
  splits, per-tensor dynamic scaling, the amax history.
* "Accelerate LLM training with NVFP4 on Blackwell" (setupai digest) --
  "Technical deep-dive": E2M1 values in about -6..6, the two-level NVFP4
  scaling (one E4M3 scale per 16 values plus one FP32 scale per tensor),
  about 4.5 bits per value.
* "How to optimize Transformer-based models for low-precision training"
  (NVIDIA blog) -- "Model configuration and training inputs",
  "Using autocast mode vs pre-quantized mode", "Interpreting results for a
  real model": the CodonFM-5B shapes, the 12 GEMMs, random Hadamard
  transform on the Wgrad inputs, stochastic rounding of gradients, 2D block
  scaling of weights, the extra per-tensor amax pass.
* "Faster training throughput in FP8 precision with NVIDIA NeMo" (NVIDIA
  blog) -- "What are the strengths and trade-offs of the FP8 scaling
  recipes?", "Scaling recipe granularity": delayed vs current per-tensor
  scaling, 1x128 / 128x128 sub-channel blocks, MXFP8 with 32-value blocks
  and E8M0 power-of-two scales.

Modules:
  formats   -- E4M3, E5M2, E8M0, E2M1 codecs by table enumeration.
  philox    -- Philox4x32-10 (Salmon et al., SC'11).
  recipes   -- amax, scales, casts for every recipe, RHT16, SR.
  gemm_ref  -- fp64 GEMM over dequantized operands and its error bound.
  passes    -- which quantized copy each Fprop / Dgrad / Wgrad GEMM consumes.

Where the pages are silent the oracle takes one reading, stated at the
function that implements it.  Every function is pinned in the tests by
something other than itself: PyTorch's float8 dtypes, exact rational
arithmetic, brute force over tiny inputs, closed forms, rocRAND's
header-only Philox4x32-10, or the facts the pages print.  Two choices are
readings that no outside fact can pin, and the tests pin them only as
stated: the order of the RHT butterfly stages (1, 2, 4, 8), and the order
of the two roundings in the NVFP4 block scale (divide by 6, then multiply).
"""
