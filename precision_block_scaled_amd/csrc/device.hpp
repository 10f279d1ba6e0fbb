// Device helpers for the gfx950 kernels: bf16 access, the bit-level E4M3
// encoder of NVFP4 block scales, E8M0 exponent selection, Philox4x32-10,
// stochastic rounding and the 16-point random Hadamard transform.
//
// The E4M3 encoder works on the bits of an IEEE binary32 value: the
// rounding of the value into the narrow format is a round-to-nearest-even
// right shift of (exponent | mantissa), which carries into the exponent by
// itself.  Saturation is a compare against the bit pattern of the largest
// finite value.  (Element codes are produced by the hardware conversion
// instructions, see the cast kernels.)  Formats: "Optimizing Transformer models for low-precision
// training", "Technical deep-dive" (E4M3 / E5M2 bit splits); "Accelerate LLM
// training with NVFP4 on Blackwell", "Technical deep-dive" (E2M1, values in
// -6..6).  Rounding rule where the pages are silent: nearest, ties to even,
// saturating, sign of zero kept.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pbs {

typedef uint16_t bf16_t;

__device__ __forceinline__ float bf16_to_float(uint32_t b) { return __uint_as_float(b << 16); }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (non-temporal: the data is read once).
__device__ __forceinline__ uint4 ld_nt16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// MXFP8 block exponent: E8M0 code of the smallest e in [-127, 127] with
// amax <= 448 * 2^e, from the bf16 bits of a non-negative block maximum.
// amax = 1.f * 2^(E-127): e = E - 135 if f <= 0.75, else E - 134.
// Zero, bf16 subnormals and anything below 448 * 2^-127 give code 0.
__device__ __forceinline__ uint32_t mx_e8m0_from_bf16_amax(uint32_t abits) {
  int E = (int)((abits >> 7) & 0xFFu);
  if (E == 0) return 0u;
  int c = E - 8 + (((abits & 0x7Fu) > 0x60u) ? 1 : 0);
  c = c < 0 ? 0 : (c > 254 ? 254 : c);
  return (uint32_t)c;
}

// MXFP4 E8M0 code from the fp32 bits of a block maximum a (sign clear):
// the smallest e in [-127, 127] with a <= 6 * 2^e.  With a = m * 2^E, m in
// [1, 2): e = E - 2 if m <= 1.5, else E - 1; zero and fp32 subnormals give
// the clamp -127.  Returns c = e + 127.
__device__ __forceinline__ uint32_t mx4_e8m0_from_f32_amax(uint32_t abits) {
  const int E = (int)(abits >> 23);
  int c = E - 2 + (((abits & 0x7FFFFFu) > 0x400000u) ? 1 : 0);
  c = c < 0 ? 0 : (c > 254 ? 254 : c);
  return (uint32_t)c;
}

// 2^(127 - c) as float for an E8M0 code c in [0, 254]: the factor that
// divides a block by its scale.  Normal for every c that can occur (c <= 247).
__device__ __forceinline__ float mx_inv_scale(uint32_t c) {
  return __uint_as_float((254u - c) << 23);
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC'11): ten rounds of two 32x32->64 products and a
// word permutation, key bumped by the Weyl constants between rounds.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                               uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    // one 32x32->64 product each (v_mad_u64_u32), not separate lo / hi halves
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c0 = n0; c1 = (uint32_t)p1; c2 = n2; c3 = (uint32_t)p0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return make_uint4(c0, c1, c2, c3);
}

__device__ __forceinline__ uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                                 uint32_t k1) {
  return philox4x32_10(c0, c1, c2, c3, k0, k1).x;
}

// Stochastic-rounding words: logical element i of x (row-major index
// r * C + c) takes word i % 4 of the call with counter (i / 4, 0, 0), so four
// consecutive elements of a row share one call.  sr_words4(q) is the call
// for elements 4 q .. 4 q + 3, sr_word(i) one element's word.
__device__ __forceinline__ uint4 sr_words4(uint64_t q, uint64_t seed) {
  return philox4x32_10((uint32_t)q, (uint32_t)(q >> 32), 0u, 0u, (uint32_t)seed, (uint32_t)(seed >> 32));
}

__device__ __forceinline__ uint32_t sr_word(uint64_t i, uint64_t seed) {
  const uint4 w = sr_words4(i >> 2, seed);
  const uint32_t k = (uint32_t)i & 3u;
  return k == 0 ? w.x : k == 1 ? w.y : k == 2 ? w.z : w.w;
}

// Stochastic rounding of v to E2M1 with the 32-bit random r: |v| >= 6 gives
// 6; otherwise with lo <= |v| < hi adjacent E2M1 magnitudes, round up iff
// r < ceil((|v| - lo) / (hi - lo) * 2^32).  Computed on the fp32 bit pattern
// ua of |v|, exactly: from 1 up, an E2M1 step covers the upper or lower half
// of a binade (steps 0.5, 1, 2 in [1, 2), [2, 4), [4, 8)), so lo's code is
// (ua >> 22) - 252 and the position within the step is the 22 mantissa bits
// below the halving bit, i.e. the threshold is ua << 10 (mod 2^32); in
// [0.5, 1) lo = 0.5 (code 1) and the position is the whole 23-bit mantissa,
// ua << 9; below 0.5 lo = 0 and the threshold is ceil(|v| * 2^33), exact in
// fp32.  A NaN saturates like |v| >= 6 (the code above 6's bit pattern),
// as the oracle's rule does.
__device__ __forceinline__ uint32_t sr_e2m1(float v, uint32_t r) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t ua = u & 0x7FFFFFFFu;
  const uint32_t sign = (u >> 28) & 0x8u;
  const bool ge1 = ua >= 0x3F800000u, ge05 = ua >= 0x3F000000u;
  const uint32_t lo = ge1 ? (ua >> 22) - 252u : (ge05 ? 1u : 0u);
  const uint32_t T =
      ge1 ? (ua << 10) : (ge05 ? (ua << 9) : (uint32_t)ceilf(__uint_as_float(ua) * 8589934592.0f));
  const uint32_t code = ua >= 0x40C00000u ? 7u : lo + (r < T ? 1u : 0u);
  return sign | code;
}

// 16-point random Hadamard transform of u[0..15] (in place):
// y = 1/4 * H16 * D * x with D = diag(sign bits), Sylvester-ordered H16,
// butterfly stages h = 1, 2, 4, 8, each an fp32 add and subtract, then an
// exact multiply by 0.25.  sign_mask bit j set means sigma_j = -1.
__device__ __forceinline__ void rht16(float* u, uint32_t sign_mask) {
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if ((sign_mask >> j) & 1u) u[j] = -u[j];
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & h) == 0) {
        float a = u[i], b = u[i + h];
        u[i] = a + b;
        u[i + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) u[j] = u[j] * 0.25f;
}

// Sign mask of the RHT: bit j = bit 0 of word 0 of Philox(key = seed,
// counter = (j, 0, 1, 0)).
__device__ __forceinline__ uint32_t rht_sign_mask(uint64_t seed) {
  uint32_t m = 0;
  for (uint32_t j = 0; j < 16; ++j)
    m |= (philox_word0(j, 0u, 1u, 0u, (uint32_t)seed, (uint32_t)(seed >> 32)) & 1u) << j;
  return m;
}

// fp32 scale = fmax / a with the corner rules: a == 0 -> 1, overflow -> FLT_MAX.
__device__ __forceinline__ float scale_from_amax(float a, float fmax) {
  if (a == 0.0f) return 1.0f;
  float s = fmax / a;
  return (__float_as_uint(s) == 0x7F800000u) ? 3.40282346638528859812e+38f : s;
}

}  // namespace pbs
