/*
 * pbs.h -- block-scaled quantize-then-GEMM for the linear layers of a
 * Transformer, on AMD Instinct MI355X (gfx950).  C ABI of libpbs.so.
 *
 * What the library computes follows these pages:
 *  [LP]  "How to optimize Transformer-based models for low-precision
 *        training" (NVIDIA technical blog).
 *  [NEMO] "Faster training throughput in FP8 precision with NVIDIA NeMo"
 *        (NVIDIA technical blog).
 *  [OPT] "Optimizing Transformer models for low-precision training"
 *        (setupai.cc digest of an NVIDIA blog post).
 *  [FP4] "Accelerate LLM training with NVFP4 on Blackwell" (setupai.cc
 *        digest of an NVIDIA blog post).
 * Each entry point names the section it implements.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Pointers are DEVICE pointers unless marked [host].  The caller owns
 *    every buffer; the library never allocates or frees device memory and
 *    keeps no device state between calls.
 *  - Every call only enqueues work on `stream` (a hipStream_t; 0 = the
 *    null stream) and returns without synchronising.  Outputs are valid
 *    once the stream reaches that point.
 *  - Arguments are validated on the host before anything is enqueued; on
 *    a validation error nothing is enqueued.  A failed kernel launch
 *    returns PBS_ERR_HIP.  pbs_last_error() gives a text message for the
 *    calling thread's last failure.  No C++ exception crosses the ABI.
 *  - There is no silent fallback ([LP], "Interpreting results for a real
 *    model", warns that an unsupported layer can fall back to a wider
 *    format unnoticed): a combination without a kernel returns
 *    PBS_ERR_UNSUPPORTED.  Setting the environment variable
 *    PBS_LOG_LEVEL=1 prints one line per dispatched kernel to stderr.
 *  - Tensors are row-major.  bf16 inputs are raw bf16 bit patterns.
 *  - Identical inputs give identical output bytes (amax reductions use an
 *    order-independent maximum).
 *  - Shapes: every dimension that a block runs along must be a multiple
 *    of that block (16, 32 or 128), every cast dimension a multiple of 16,
 *    and GEMM dimensions as stated at pbs_gemm; otherwise PBS_ERR_SHAPE.
 */
#ifndef PBS_H
#define PBS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PBS_VERSION 4   /* 3: pbs_rht_cast, pbs_debug_sr_encode; 4: four SR words per Philox call */

typedef enum {
  PBS_OK = 0,
  PBS_ERR_INVALID_ARG = 1, /* null pointer, unknown enum, bad flag         */
  PBS_ERR_SHAPE = 2,       /* dimension not a multiple of block / tile     */
  PBS_ERR_UNSUPPORTED = 3, /* recipe / format / layout with no kernel      */
  PBS_ERR_HIP = 4          /* a HIP launch or runtime call failed          */
} pbs_status;

/* Element formats.  E4M3 is the OCP "FN" variant (max 448, no Inf); E5M2
 * max 57344; E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 ([OPT] "Technical
 * deep-dive"; [FP4] "Technical deep-dive"). */
typedef enum {
  PBS_FMT_BF16 = 0,
  PBS_FMT_E4M3 = 1,
  PBS_FMT_E5M2 = 2,
  PBS_FMT_E2M1 = 3,
  PBS_FMT_F32 = 4
} pbs_format;

/* Scaling recipes ([NEMO] "What are the strengths and trade-offs of the
 * FP8 scaling recipes?", "Scaling recipe granularity"; [FP4] "Technical
 * deep-dive"). */
typedef enum {
  PBS_RECIPE_BF16 = 0,         /* no quantization: bf16 operands            */
  PBS_RECIPE_FP8_CURRENT = 1,  /* per-tensor scale from this tensor's amax  */
  PBS_RECIPE_FP8_DELAYED = 2,  /* per-tensor scale from an amax history     */
  PBS_RECIPE_FP8_BLOCK128 = 3, /* fp32 scale per 1x128 (act/grad) or
                                  128x128 (weight) block, E4M3 values       */
  PBS_RECIPE_MXFP8 = 4,        /* E8M0 scale per 32 values, E4M3 values     */
  PBS_RECIPE_NVFP4 = 5,        /* E2M1 values, E4M3 scale per 16 values (1x16
                                  act/grad, 16x16 weight), fp32 per tensor  */
  PBS_RECIPE_MXFP4 = 6,        /* E2M1 values, E8M0 scale per 32 values     */
  PBS_RECIPE_FP8_CHANNEL = 7,  /* fp32 scale per row of each copy (per
                                  channel), E4M3 values                     */
  PBS_RECIPE_FP8_BLOCK128_1D1D = 8, /* as FP8_BLOCK128 with 1x128 blocks on
                                  every tensor, weights included           */
  PBS_RECIPE_FP8_BLOCK128_2D2D = 9, /* as FP8_BLOCK128 with 128x128 blocks on
                                  every tensor                              */
  PBS_RECIPE_FP8_BLOCK128_POW2 = 10 /* FP8_BLOCK128's blocks with power-of-two
                                  (E8M0) scales, E4M3 values                */
} pbs_recipe;

/* The three GEMMs of a linear layer ([LP] "Using autocast mode vs
 * pre-quantized mode": Fprop, Dgrad and Wgrad are timed separately).
 * With X [M_tok, K_in], W stored [N_out, K_in], dY [M_tok, N_out]:
 *   FPROP  Y  [M_tok, N_out] = X  . W^T   contraction K_in
 *   DGRAD  dX [M_tok, K_in]  = dY . W     contraction N_out
 *   WGRAD  dW [K_in, N_out]  = X^T . dY   contraction M_tok              */
typedef enum { PBS_FPROP = 0, PBS_DGRAD = 1, PBS_WGRAD = 2 } pbs_layout;

/* Orientation of a quantized copy.  ROW: blocks run along the stored
 * columns, output has the input's shape [rows, cols].  COL: blocks run
 * along the stored rows and the output is written transposed,
 * [cols, rows], so that in both cases the blocks run along the output's
 * contiguous axis (the GEMM contraction axis). */
#define PBS_ROW 1
#define PBS_COL 2

/* Cast / amax flags. */
#define PBS_FLAG_RHT16 1   /* apply the 16x16 random Hadamard transform along
                              the rows first (NVFP4 / MXFP4 Wgrad operands) */
#define PBS_FLAG_SR 2      /* stochastic rounding of the E2M1 values
                              (NVFP4 / MXFP4 gradients)                     */

/* ---------------------------------------------------------------------
 * pbs_amax: amax_out[0] = max |x| over a bf16 tensor [rows, cols].
 * [OPT] "Technical deep-dive" (per-tensor dynamic scaling from the max
 * absolute value); [LP] "Interpreting results for a real model" (NVFP4's
 * extra per-tensor amax pass).  With PBS_FLAG_RHT16 the maximum is taken
 * over the float32 result of the random Hadamard transform applied along
 * the rows (rows % 16 == 0), sign seed `seed`.  The result is exact.
 * amax_out: 1 float, overwritten (no need to clear it first).
 * ------------------------------------------------------------------- */
pbs_status pbs_amax(const void* x_bf16, int64_t rows, int64_t cols, int flags,
                    uint64_t seed, float* amax_out, hipStream_t stream);

/* ---------------------------------------------------------------------
 * pbs_scale_from_amax: scale[0] = fp32(fmax / amax[0]), scale_inv[0] =
 * fp32(1 / scale[0]); amax 0 gives scale 1, an overflowing division gives
 * FLT_MAX.  fmax = 448 (E4M3), 57344 (E5M2), or 2688 (= 6 * 448, the NVFP4
 * per-tensor encode scale S_enc; scale_inv is then S_dec).
 * [NEMO] per-tensor current scaling item; [FP4] two-level scaling.
 * Any of scale / scale_inv may be NULL.
 * ------------------------------------------------------------------- */
pbs_status pbs_scale_from_amax(const float* amax, float fmax, float* scale,
                               float* scale_inv, hipStream_t stream);

/* ---------------------------------------------------------------------
 * Delayed scaling state ([OPT] "Technical deep-dive": a rolling amax
 * history, scale from earlier iterations; [NEMO] per-tensor delayed
 * scaling item).  The state is a caller-owned device buffer of
 * pbs_delayed_state_bytes() bytes; checkpointing it is a plain copy.
 * Layout: float scale; float scale_inv; int32 pos; int32 len;
 *         float history[len].
 *  init:   history = 0, pos = 0, scale = scale_inv = 1.
 *  A step: pbs_cast(PBS_RECIPE_FP8_DELAYED, scale = pbs_delayed_scale(st),
 *          amax_out = a) casts with the current scale and measures the
 *          tensor's amax in the same pass; the GEMM of the step reads
 *          pbs_delayed_scale_inv(st); then
 *  update: history[pos] = a[0]; pos = (pos + 1) % len;
 *          scale = fp32(fmax / max(history)) (1 if 0, FLT_MAX on overflow);
 *          scale_inv = fp32(1 / scale).
 * Enqueue the GEMM that consumes a delayed cast before the update.
 * ------------------------------------------------------------------- */
pbs_status pbs_delayed_state_bytes(int hist_len, size_t* bytes /* [host] */);
pbs_status pbs_delayed_init(void* state, int hist_len, hipStream_t stream);
pbs_status pbs_delayed_update(void* state, const float* amax, float fmax,
                              hipStream_t stream);
float* pbs_delayed_scale(void* state);     /* device address of `scale`     */
float* pbs_delayed_scale_inv(void* state); /* device address of `scale_inv` */

/* ---------------------------------------------------------------------
 * pbs_cast: quantize a bf16 tensor x [rows, cols] into a row copy, a col
 * copy, or both from one read (orient_mask = PBS_ROW | PBS_COL).
 *
 *  recipe FP8_CURRENT / FP8_DELAYED ([NEMO] per-tensor items):
 *    fmt E4M3 or E5M2; scale = device fp32 scalar s; codes =
 *    enc(fp32(x * s)), round-to-nearest-even, saturating.  No block
 *    scales (row_scales / col_scales ignored).  amax_out (optional, may be
 *    NULL): receives max |x|, measured in the same pass (delayed scaling).
 *  recipe FP8_BLOCK128 ([NEMO] "Scaling recipe granularity"): fmt E4M3;
 *    weight_2d = 0: one scale per 1x128 block along the contraction axis,
 *    scales [rows, cols/128] (row copy) / [cols, rows/128] (col copy);
 *    weight_2d = 1: one scale per 128x128 tile, [rows/128, cols/128] /
 *    [cols/128, rows/128].  Stored scale = fp32(1 / s_b), s_b =
 *    fp32(448 / amax_b).  `scale` unused.
 *  recipes FP8_BLOCK128_1D1D / FP8_BLOCK128_2D2D ([NEMO] "Scaling recipe
 *    granularity": the other block pairings, read as (activations and
 *    gradients, weights) with 1D = 1x128 and 2D = 128x128): the same cast;
 *    the caller passes weight_2d = 0 for every tensor (1D1D) or 1 for every
 *    tensor (2D2D).
 *  recipe FP8_BLOCK128_POW2 ([NEMO] "Scaling recipe granularity" for the
 *    blocks, its MXFP8 item for the power-of-two scale): fmt E4M3; the
 *    blocks of FP8_BLOCK128 (weight_2d selects 128x128), each with MXFP8's
 *    exponent rule (smallest e in [-127, 127] with amax_b <= 448 * 2^e,
 *    codes = enc(x * 2^-e)).  Each block's scale is stored as one 32-bit
 *    word holding its E8M0 code e + 127 in all four bytes (the 4 bytes per
 *    block FP8_BLOCK128 stores, in the form the scaled matrix instruction
 *    reads per 32-value step): uint32 [rows, cols/128] / [cols, rows/128],
 *    or [rows/128, cols/128] / [cols/128, rows/128] with weight_2d = 1.
 *    Scales 4-byte aligned.  `scale` unused.
 *  recipe MXFP8 ([NEMO] MXFP8 item): fmt E4M3, 32-value blocks along the
 *    contraction axis, E8M0 scale bytes [rows, cols/32] / [cols, rows/32];
 *    the exponent is the smallest e with amax_b <= 448 * 2^e.
 *  recipe NVFP4 ([FP4] "Technical deep-dive"; [LP] "Interpreting results
 *    for a real model"): fmt E2M1, codes packed two per byte along the
 *    contiguous axis, even element in the low nibble: [rows, cols/2] /
 *    [cols, rows/2].  E4M3 block scale bytes per 1x16 (weight_2d = 0) or
 *    16x16 (weight_2d = 1) block, laid out like FP8_BLOCK128's with 16 for
 *    128.  scale = device fp32 S_enc (pbs_scale_from_amax with fmax 2688 of
 *    this tensor's amax, taken after the RHT when it is used).
 *    flags: PBS_FLAG_RHT16 (col copy only, rows % 16 == 0; sign seed
 *    `seed`), PBS_FLAG_SR (stochastic rounding with Philox4x32-10, key =
 *    `seed`: logical element i = r * cols + c of x takes word i % 4 of the
 *    call with counter (i / 4, 0, 0)).
 *  recipe MXFP4 ([FP4] "Technical deep-dive": the 32-value MX format that
 *    NVFP4's 16-value blocks refine): fmt E2M1, codes packed as for NVFP4;
 *    E8M0 scale bytes per 1x32 block along the contraction axis, [rows,
 *    cols/32] / [cols, rows/32]; the exponent is the smallest e with
 *    amax_b <= 6 * 2^e (no element saturates), codes = enc_E2M1(x * 2^-e).
 *    Same flags as NVFP4 (PBS_FLAG_RHT16 col copy only, PBS_FLAG_SR).
 *    `scale` unused.
 *  recipe FP8_CHANNEL ([NEMO] "Scaling recipe granularity": per-channel
 *    scaling, between one scale per tensor and blocks): fmt E4M3; one fp32
 *    scale per row of each copy, i.e. per row of x for the row copy
 *    (row_scales [rows]) and per column of x for the col copy (col_scales
 *    [cols]); stored scale = fp32(1 / s_r), s_r = fp32(448 / amax_r) (1 for
 *    an all-zero row, FLT_MAX on overflow); codes = enc(fp32(x * s_r)).
 *    Scales 4-byte aligned.  The row copy reads x once; the col copy reads
 *    it twice (column maxima, then the cast) and uses col_scales as the
 *    running maxima in between.  `scale` unused.
 *  Outputs for an orientation not in orient_mask may be NULL.
 *  2D-block casts (weight_2d = 1) and two-copy casts with stochastic
 *  rounding take at most 65535 x 128 rows (else PBS_ERR_SHAPE); other 1D
 *  casts, two-copy ones included, have no such limit.
 * ------------------------------------------------------------------- */
pbs_status pbs_cast(pbs_recipe recipe, const void* x_bf16, int64_t rows, int64_t cols,
                    pbs_format fmt, int orient_mask, int weight_2d, int flags,
                    uint64_t seed, const float* scale, float* amax_out,
                    void* row_codes, void* row_scales, void* col_codes,
                    void* col_scales, hipStream_t stream);

/* ---------------------------------------------------------------------
 * pbs_rht_cast: the transposed (col) copy of a Wgrad operand of the 4-bit
 * recipes, with the 16x16 random Hadamard transform applied first along
 * the rows and, optionally, stochastic rounding of the E2M1 values ([LP]
 * "Interpreting results for a real model": NVFP4 applies a random Hadamard
 * transform to the Wgrad inputs and rounds gradients stochastically; [FP4]
 * "Technical deep-dive": the two-level NVFP4 scaling).
 *  recipe: PBS_RECIPE_NVFP4 or PBS_RECIPE_MXFP4.  x bf16 [rows, cols],
 *    rows % 16 == 0 (each 16-row group of a column is transformed).
 *  rht_seed: Philox4x32-10 key of the signs (sigma_j = bit 0 of word 0 of
 *    Philox(counter (j, 0, 1, 0))), the same key as pbs_amax's seed for the
 *    transformed maximum.
 *  stochastic = 1: stochastic rounding with key sr_seed, words as for
 *    pbs_cast's PBS_FLAG_SR (element i = r * cols + c of x: word i % 4 of
 *    the call with counter i / 4); 0: round to nearest even (sr_seed
 *    unused).
 *  scale: NVFP4's device fp32 S_enc (pbs_scale_from_amax, fmax 2688, of
 *    the transformed tensor's amax); unused for MXFP4.
 *  col_codes [cols, rows / 2] packed E2M1, col_scales E4M3 [cols, rows / 16]
 *    (NVFP4) or E8M0 [cols, rows / 32] (MXFP4), as pbs_cast's col copy.
 *  pbs_cast(recipe, ..., PBS_COL, 0, PBS_FLAG_RHT16 | PBS_FLAG_SR, seed, ...)
 *  is this call with rht_seed = sr_seed = seed.  Errors as pbs_cast.
 * ------------------------------------------------------------------- */
pbs_status pbs_rht_cast(pbs_recipe recipe, const void* x_bf16, int64_t rows, int64_t cols,
                        uint64_t rht_seed, int stochastic, uint64_t sr_seed, const float* scale,
                        void* col_codes, void* col_scales, hipStream_t stream);

/* ---------------------------------------------------------------------
 * pbs_gemm: C[M, N] = sum_k A[m, k] * B[n, k] with fp32 accumulation, in
 * the GEMM of `layout` ([LP] "Model configuration and training inputs":
 * every linear layer is an M x K x N product; "Using autocast mode vs
 * pre-quantized mode": Fprop / Dgrad / Wgrad).  M, N, K are the GEMM's own
 * dims (output rows, output cols, contraction).
 *
 * Quantized recipes: A is [M, K] and B is [N, K], both contraction-
 * contiguous, i.e. the copies pbs_cast produces:
 *   FPROP: A = X row copy,  B = W row copy
 *   DGRAD: A = dY row copy, B = W col copy
 *   WGRAD: A = X col copy,  B = dY col copy
 *  - FP8_CURRENT / FP8_DELAYED: a_fmt, b_fmt in {E4M3, E5M2};
 *    a_tensor_scale / b_tensor_scale = device fp32 scale_inv of each
 *    operand; C = acc * fp32(sa_inv * sb_inv).
 *  - FP8_BLOCK128: a_scale = fp32 [M, K/128]; b_scale = fp32 [N/128, K/128]
 *    for FPROP / DGRAD (weights, 2D) or [N, K/128] for WGRAD; each 128-long
 *    slice of the contraction is accumulated apart and added in with the
 *    product of its two scales.
 *  - FP8_BLOCK128_1D1D: a_scale = fp32 [M, K/128], b_scale = fp32
 *    [N, K/128] in every pass.
 *  - FP8_BLOCK128_2D2D: a_scale = fp32 [M/128, K/128], b_scale = fp32
 *    [N/128, K/128] in every pass; M and N multiples of 128.
 *  - MXFP8: a_scale = E8M0 [M, K/32], b_scale = E8M0 [N, K/32].
 *  - FP8_BLOCK128_POW2: a_scale = uint32 [M, K/128] (pbs_cast's E8M0 words);
 *    b_scale = uint32 [N/128, K/128] for FPROP / DGRAD (weights, 2D) or
 *    [N, K/128] for WGRAD; 4-byte aligned.  The power-of-two scales are
 *    applied by the matrix instruction itself, as for MXFP8.
 *  - NVFP4: A, B packed E2M1 [M, K/2], [N, K/2]; a_scale = E4M3 [M, K/16];
 *    b_scale = E4M3 [N/16, K/16] for FPROP / DGRAD (weights, 2D) or
 *    [N, K/16] for WGRAD; a_tensor_scale / b_tensor_scale = S_dec of each.
 *  - MXFP4: A, B packed E2M1 [M, K/2], [N, K/2]; a_scale = E8M0 [M, K/32],
 *    b_scale = E8M0 [N, K/32]; tensor scales unused.
 *  - FP8_CHANNEL: a_fmt = b_fmt = E4M3; a_scale = fp32 [M] and b_scale =
 *    fp32 [N] (the stored scale of each operand row, pbs_cast's channel
 *    scales), 16-byte aligned; C[m, n] = acc * fp32(a_scale[m] *
 *    b_scale[n]); tensor scales unused.
 * BF16 recipe: operands in their natural storage -- FPROP: A = X [M, K],
 *    B = W [N, K]; DGRAD: A = dY [M, K], B = W stored [K, N]; WGRAD:
 *    A = X stored [K, M], B = dY stored [K, N].
 * c_fmt: PBS_FMT_F32 or PBS_FMT_BF16 (round-to-nearest-even).
 * Shapes (else PBS_ERR_SHAPE): M, N multiples of 16 (ragged 256-tiles are
 *   masked); K a multiple of 128 (FP8 recipes, NVFP4), 256 (MXFP4) or 64
 *   (BF16); each stored operand row at most 16 MiB.  K == 0 writes zeros
 *   to C.
 * Alignment (else PBS_ERR_INVALID_ARG): A, B, C 16-byte aligned; MXFP8,
 *   MXFP4, NVFP4 and FP8_BLOCK128_POW2 block scales 4-byte aligned;
 *   FP8_CHANNEL scales
 *   16-byte aligned.
 * Accuracy: fp32 accumulation; the 8-bit instructions (FP8 recipes) truncate
 *   each product of an aligned group of 8 toward zero to a multiple of
 *   2^(e - 13), e the group's largest sum of operand exponents, and add the
 *   exact sum of two such groups to the fp32 accumulator with one rounding
 *   to nearest even; BF16 and NVFP4 (decoded exactly to fp16 in registers)
 *   accumulate at fp32 precision; MXFP4 uses the same instruction as the
 *   FP8 recipes with E2M1 inputs (whose products it keeps exactly).
 * C is overwritten; calls on one stream are ordered, nothing is allocated.
 * ------------------------------------------------------------------- */
pbs_status pbs_gemm(pbs_recipe recipe, pbs_layout layout, int64_t M, int64_t N, int64_t K,
                    const void* A, pbs_format a_fmt, const void* a_scale,
                    const float* a_tensor_scale, const void* B, pbs_format b_fmt,
                    const void* b_scale, const float* b_tensor_scale, void* C,
                    pbs_format c_fmt, hipStream_t stream);

/* ---------------------------------------------------------------------
 * pbs_gemm_amax: pbs_gemm that also returns max |C| over the stored output
 * ([LP] "Interpreting results for a real model" counts the extra memory
 * pass for the per-tensor maximum among the quantization overheads; a
 * tensor that a GEMM produces gets its maximum from the GEMM's epilogue
 * instead, with no second read of C).
 *  c_amax: device fp32, receives max |C| of the values as stored (after
 *    the epilogue scale and, for bf16 output, after rounding to bf16), i.e.
 *    what pbs_amax would return on C; reset to 0 first (stream-ordered), 0
 *    for an empty C.  Must be non-null and 4-byte aligned (else
 *    PBS_ERR_INVALID_ARG); the other arguments and errors are pbs_gemm's,
 *    and C is bit-identical to pbs_gemm's.
 * ------------------------------------------------------------------- */
pbs_status pbs_gemm_amax(pbs_recipe recipe, pbs_layout layout, int64_t M, int64_t N, int64_t K,
                         const void* A, pbs_format a_fmt, const void* a_scale,
                         const float* a_tensor_scale, const void* B, pbs_format b_fmt,
                         const void* b_scale, const float* b_tensor_scale, void* C,
                         pbs_format c_fmt, float* c_amax, hipStream_t stream);

/* ---------------------------------------------------------------------
 * pbs_quantized_bytes [host]: bytes of the codes and of the block scales
 * of one quantized copy of a [rows, cols] tensor (not counting per-tensor
 * fp32 scalars).  For NVFP4 with 1x16 blocks this is n/2 + n/16 bytes,
 * about 4.5 bits per value with the fp32 tensor scale ([FP4] "Technical
 * deep-dive").
 * ------------------------------------------------------------------- */
pbs_status pbs_quantized_bytes(pbs_recipe recipe, int64_t rows, int64_t cols, int weight_2d,
                               size_t* code_bytes, size_t* scale_bytes);

/* ---------------------------------------------------------------------
 * pbs_debug_sr_encode: test hook.  codes[i] = the device's stochastic
 * E2M1 rounding of v[i] with the 32-bit random word r[i] (4-bit code, sign
 * in bit 3, one per byte), the rule every SR cast applies ([LP]
 * "Interpreting results for a real model": stochastic rounding of
 * gradients): |v| >= 6 gives 6; otherwise, with lo <= |v| < hi adjacent
 * E2M1 magnitudes, hi iff r < ceil((|v| - lo) / (hi - lo) * 2^32), else
 * lo; the sign of v is kept.  v fp32 and r uint32 (4-byte aligned), codes
 * uint8, n values; n == 0 enqueues nothing.
 * ------------------------------------------------------------------- */
pbs_status pbs_debug_sr_encode(const float* v, const uint32_t* r, uint8_t* codes, int64_t n,
                               hipStream_t stream);

const char* pbs_last_error(void);
int pbs_version(void);

#ifdef __cplusplus
}
#endif
#endif /* PBS_H */
