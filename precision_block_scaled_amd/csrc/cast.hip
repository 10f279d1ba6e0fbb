// Quantize (cast) kernels for every recipe.
//
// Four kernel templates, each instantiated per recipe:
//   * cast_row_kernel: the row copy with 1D blocks (every GEMM operand but
//     2D-blocked weights): a lane quantizes 8 consecutive values at a time,
//     no LDS;
//   * cast_rc_kernel: the transposed (col) copy with 1D blocks, alone or
//     with the row copy from the same read, through a 256 x 128 tile in LDS;
//   * cast_col_kernel: the col copy with the Hadamard transform or
//     stochastic rounding, through a 256 x 64 tile in LDS;
//   * cast_tile_kernel: 2D weight blocks, and both copies from one read
//     with stochastic rounding.  A workgroup of 128 threads stages a 128 x 128 tile of
//     the bf16 input in LDS, then thread t quantizes row t of the tile
//     (row copy, blocks along the columns) and/or column t (col copy, written
//     as row t of the transposed output), so every 1D block (16, 32 or 128
//     long) lies inside one thread's strip; 16x16 NVFP4 blocks reduce across
//     16 neighbouring lanes and 128x128 blocks use the tile maximum.
// Channel-wise FP8 has its own row and column-maximum kernels (below).
//
// Recipes:
//  per-tensor FP8 -- "Faster training throughput in FP8 precision with NVIDIA
//    NeMo", strengths and trade-offs (per-tensor current / delayed items);
//    codes = enc(fp32(x * s)).
//  sub-channel FP8 -- same page, "Scaling recipe granularity": 1x128 blocks
//    for activations and gradients, 128x128 for weights; s_b = fp32(448 /
//    amax_b), stored as fp32(1 / s_b).
//  MXFP8 -- same page, MXFP8 item: 32-value blocks, E8M0 power-of-two scale,
//    the smallest exponent that brings the block maximum within 448.
//  sub-channel FP8 with power-of-two scales -- the sub-channel blocks with
//    MXFP8's exponent rule; each block's E8M0 code is stored in all four
//    bytes of a 32-bit word (the form the scaled matrix instruction reads).
//  NVFP4 -- "Accelerate LLM training with NVFP4 on Blackwell", "Technical
//    deep-dive": E2M1 values, E4M3 scale per 16 values, fp32 per tensor;
//    "How to optimize Transformer-based models for low-precision training",
//    "Interpreting results for a real model": 2D block scales for weights,
//    random Hadamard transform on the Wgrad inputs, stochastic rounding of
//    gradients.  d = enc_E4M3(fp32(fp32(amax_b / 6) * S_enc)), e_b =
//    fp32(S_enc / d), codes = enc_E2M1(fp32(x * e_b)) or its stochastic
//    rounding with Philox4x32-10 (logical element i takes word i % 4 of the
//    call with counter i / 4).
//  channel-wise FP8 -- "Faster training throughput in FP8 precision with
//    NVIDIA NeMo", "Scaling recipe granularity" (per-channel scaling): one
//    scale per row of each contraction-contiguous copy, s_r = fp32(448 /
//    amax_r) with the per-tensor corner rules, stored as fp32(1 / s_r).
//  MXFP4 -- "Accelerate LLM training with NVFP4 on Blackwell", "Technical
//    deep-dive" (the 32-value MX format NVFP4 refines): E2M1 values, E8M0
//    power-of-two scale per 32, the smallest exponent that brings the block
//    maximum within 6; the Hadamard transform and stochastic rounding as for
//    NVFP4.
#include "device.hpp"
#include "host.hpp"

#include <algorithm>

namespace pbs {

enum { R_TENSOR = 0, R_BLOCK128 = 1, R_MX = 2, R_NV = 3, R_MX4 = 4, R_CHAN = 5, R_B128P2 = 6 };
enum { F_E4M3 = 0, F_E5M2 = 1 };

constexpr int TILE = 128;
constexpr int LDS_STRIDE = TILE + 8;   // bf16 per LDS row: 272 B, offsets rows by 4 banks

struct CastArgs {
  const bf16_t* x;
  int64_t R, C;
  const float* scale;      // per-tensor s, or NVFP4 S_enc
  uint32_t* amax_out;      // fused amax (per-tensor recipes), may be null
  uint8_t* row_codes;
  void* row_scales;
  uint8_t* col_codes;
  void* col_scales;
  uint64_t seed;           // Philox key of stochastic rounding
  uint64_t rht_seed;       // Philox key of the Hadamard transform's signs
};

__device__ __forceinline__ uint32_t lds_bits(const bf16_t* tile, int r, int c) {
  return (uint32_t)tile[r * LDS_STRIDE + c];
}

// 16 consecutive values of a strip: along a row (ROWDIR) or down a column.
template <bool ROWDIR>
__device__ __forceinline__ void read16(const bf16_t* tile, int strip, int off, uint32_t* b) {
  if (ROWDIR) {
    const uint4 v0 = *(const uint4*)&tile[strip * LDS_STRIDE + off];
    const uint4 v1 = *(const uint4*)&tile[strip * LDS_STRIDE + off + 8];
    const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      b[2 * i] = w[i] & 0xFFFFu;
      b[2 * i + 1] = w[i] >> 16;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) b[i] = lds_bits(tile, off + i, strip);
  }
}

__device__ __forceinline__ uint32_t max_abs_bits16(const uint32_t* b) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint32_t a = b[i] & 0x7FFFu;
    m = m > a ? m : a;
  }
  return m;
}

__device__ __forceinline__ uint2 pack_e2m1_16(const uint32_t* q) {
  uint2 w;
  w.x = q[0] | (q[1] << 4) | (q[2] << 8) | (q[3] << 12) | (q[4] << 16) | (q[5] << 20) |
        (q[6] << 24) | (q[7] << 28);
  w.y = q[8] | (q[9] << 4) | (q[10] << 8) | (q[11] << 12) | (q[12] << 16) | (q[13] << 20) |
        (q[14] << 24) | (q[15] << 28);
  return w;
}

// Max over aligned groups of G lanes.  Within a 16-lane row the exchanges
// are DPP moves (vector ALU, no LDS permute): quad_perm [1,0,3,2] and
// [2,3,0,1] reduce each quad, row_half_mirror (lane i <-> 7 - i of each
// 8-lane half) brings in the other quad of the half, row_mirror (i <-> 15 -
// i) the other half of the row.  Wider groups exchange through __shfl_xor.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max(uint32_t x) {
  const uint32_t y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
  return x > y ? x : y;
}

template <int G>
__device__ __forceinline__ uint32_t group_max(uint32_t v) {
  if (G >= 2) v = dpp_max<0xB1>(v);
  if (G >= 4) v = dpp_max<0x4E>(v);
  if (G >= 8) v = dpp_max<0x141>(v);
  if (G >= 16) v = dpp_max<0x140>(v);
#pragma unroll
  for (int o = 16; o < G; o <<= 1) {
    const uint32_t u = (uint32_t)__shfl_xor((int)v, o, 64);
    v = v > u ? v : u;
  }
  return v;
}

// Max over the 16 lanes that share bits 4..5 of the lane id.
__device__ __forceinline__ uint32_t max16lanes(uint32_t v) { return group_max<16>(v); }

// Encoding by the gfx950 conversion instructions (v_cvt_pk_fp8_f32,
// v_cvt_pk_bf8_f32, v_cvt_scalef32_pk_fp4_f32 with scale 1): they round to
// nearest even, and clamping the input to the largest finite code first
// makes them saturating.  Compared on gfx950 with bit-level software
// encoders of E4M3, E5M2 and E2M1 over every non-NaN fp32 input, they gave
// the same code every time.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Max of the 15-bit magnitudes of 8 bf16 values (one 16-byte load).
__device__ __forceinline__ uint32_t bf16_absmax8(const uint4& w) {
  const uint32_t w4[4] = {w.x, w.y, w.z, w.w};
  u16x2 m2 = {0, 0};
#pragma unroll
  for (int k = 0; k < 4; ++k) m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, w4[k] & 0x7FFF7FFFu));
  return m2.x > m2.y ? m2.x : m2.y;
}

__device__ __forceinline__ void bf16x8_to_f32(const uint4& w, float* f) {
  const uint32_t w4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f[2 * k] = __uint_as_float(w4[k] << 16);
    f[2 * k + 1] = __uint_as_float(w4[k] & 0xFFFF0000u);
  }
}

template <int FMT>
__device__ __forceinline__ uint32_t hw_fp8x4(float a, float b, float c, float d) {
  if (FMT == F_E4M3) {
    const float L = 448.0f;
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(a, -L, L), __builtin_amdgcn_fmed3f(b, -L, L), 0,
                                            false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(c, -L, L), __builtin_amdgcn_fmed3f(d, -L, L), w, true);
    return (uint32_t)w;
  } else {
    const float L = 57344.0f;
    int w = __builtin_amdgcn_cvt_pk_bf8_f32(__builtin_amdgcn_fmed3f(a, -L, L), __builtin_amdgcn_fmed3f(b, -L, L), 0,
                                            false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(__builtin_amdgcn_fmed3f(c, -L, L), __builtin_amdgcn_fmed3f(d, -L, L), w, true);
    return (uint32_t)w;
  }
}

// 8 values -> 8 E2M1 codes, element 2k in the low nibble of byte k.
__device__ __forceinline__ uint32_t hw_fp4x8(const float* v) {
#define PBS_FP4_PAIR(w, k)                                                                         \
  __builtin_amdgcn_cvt_scalef32_pk_fp4_f32((w), __builtin_amdgcn_fmed3f(v[2 * (k)], -6.0f, 6.0f),    \
                                           __builtin_amdgcn_fmed3f(v[2 * (k) + 1], -6.0f, 6.0f), 1.0f, (k))
  uint32_t w = PBS_FP4_PAIR(0u, 0);
  w = PBS_FP4_PAIR(w, 1);
  w = PBS_FP4_PAIR(w, 2);
  w = PBS_FP4_PAIR(w, 3);
#undef PBS_FP4_PAIR
  return w;
}

// NVFP4 block scale: the E4M3 code of d_val >= 0 (saturating at 448, as
// enc_E4M3 with its clamp), its exact value d, and the encode factor e_b =
// fp32(S / d) (FLT_MAX where the quotient overflows).  A block whose scale
// rounds to 0 gets e_b = 0, so its codes are the signed zeros of its values.
struct NvScale4 {
  uint32_t code;
  float e_b;
};
__device__ __forceinline__ NvScale4 nv_block_scale(float d_val, float S) {
  NvScale4 r;
  r.code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(d_val, 0.0f, 448.0f), 0.0f, 0, false) &
           0xFFu;
  const float d = __builtin_amdgcn_cvt_f32_fp8((int)r.code, 0);
  const float e_b = fminf(S / d, 3.40282346638528859812e+38f);
  r.e_b = d == 0.0f ? 0.0f : e_b;
  return r;
}

// 16 bf16 values (bit patterns) times s -> 16 FP8 codes.
template <int FMT>
__device__ __forceinline__ uint4 hw_fp8x16(const uint32_t* b, float s) {
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = bf16_to_float(b[i]) * s;
  uint4 o;
  o.x = hw_fp8x4<FMT>(v[0], v[1], v[2], v[3]);
  o.y = hw_fp8x4<FMT>(v[4], v[5], v[6], v[7]);
  o.z = hw_fp8x4<FMT>(v[8], v[9], v[10], v[11]);
  o.w = hw_fp8x4<FMT>(v[12], v[13], v[14], v[15]);
  return o;
}

// NVFP4 block: codes for 16 fp32 values with block max bits `abits`
// (of |value|), global encode scale S.  Returns the E4M3 block scale code.
template <bool SR>
__device__ __forceinline__ uint32_t nvfp4_block(const float* v, uint32_t abits, float S,
                                                const uint32_t* rnd, uint2* packed) {
  const float a_b = __uint_as_float(abits);
  const NvScale4 sc = nv_block_scale((a_b / 6.0f) * S, S);
  uint32_t q[16];
  if (sc.e_b == 0.0f) {     // the signed zeros, without the multiplies (fewer live registers under SR)
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = (__float_as_uint(v[i]) >> 28) & 0x8u;
    *packed = pack_e2m1_16(q);
  } else {
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = v[i] * sc.e_b;
    if (SR) {
#pragma unroll
      for (int i = 0; i < 16; ++i) q[i] = sr_e2m1(x[i], rnd[i]);
      *packed = pack_e2m1_16(q);
    } else {
      *packed = make_uint2(hw_fp4x8(x), hw_fp4x8(x + 8));
    }
  }
  return sc.code;
}

// Quantize one strip (a tile row if ROWDIR, else a tile column) of `len`
// valid values (multiple of 16) and write it.
//  strip: index of the strip in the tile (= thread id)
//  out_codes: start of this strip's output row segment
//  g_row/g_col of element 0 of the strip (for the SR counter)
// Stochastic-rounding words of values j .. j + N - 1 of a strip: a row strip
// (ROWDIR) of logical row g_row0 from column g_col0 (a multiple of 4, as j
// is), one call per 4 values; a column strip of column g_col0 from row
// g_row0, one call per value, whose word the column picks.
template <bool ROWDIR, int N>
__device__ __forceinline__ void sr_strip_words(const CastArgs& a, int64_t g_row0, int64_t g_col0, int j,
                                               uint32_t* rnd) {
  if (ROWDIR) {
    const uint64_t q0 = (uint64_t)(g_row0 * a.C + g_col0 + j) >> 2;
#pragma unroll
    for (int k = 0; k < N / 4; ++k) {
      const uint4 r4 = sr_words4(q0 + k, a.seed);
      rnd[4 * k] = r4.x;
      rnd[4 * k + 1] = r4.y;
      rnd[4 * k + 2] = r4.z;
      rnd[4 * k + 3] = r4.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) rnd[i] = sr_word((uint64_t)((g_row0 + j + i) * a.C + g_col0), a.seed);
  }
}

template <int RECIPE, int FMT, bool ROWDIR, bool W2D, bool RHT, bool SR>
__device__ __forceinline__ void quantize_strip(const bf16_t* tile, int strip, int len,
                                               const CastArgs& a, float tile_scale,
                                               uint8_t* out_codes, uint8_t* out_scales8,
                                               float* out_scales32, int64_t g_row0, int64_t g_col0,
                                               uint32_t rht_mask, bool scale_writer) {
  if (RECIPE == R_TENSOR) {
    const float s = tile_scale;
    for (int j = 0; j < len; j += 16) {
      uint32_t b[16];
      read16<ROWDIR>(tile, strip, j, b);
      *(uint4*)(out_codes + j) = hw_fp8x16<FMT>(b, s);
    }
  } else if (RECIPE == R_BLOCK128) {
    float s = tile_scale;
    if (!W2D) {                 // one 1x128 block = the whole strip
      uint32_t m = 0;
      for (int j = 0; j < TILE; j += 16) {
        uint32_t b[16];
        read16<ROWDIR>(tile, strip, j, b);
        uint32_t mm = max_abs_bits16(b);
        m = m > mm ? m : mm;
      }
      s = scale_from_amax(bf16_to_float(m), 448.0f);
      out_scales32[0] = 1.0f / s;
    } else if (scale_writer) {
      out_scales32[0] = 1.0f / s;
    }
    for (int j = 0; j < TILE; j += 16) {
      uint32_t b[16];
      read16<ROWDIR>(tile, strip, j, b);
      *(uint4*)(out_codes + j) = hw_fp8x16<F_E4M3>(b, s);
    }
  } else if (RECIPE == R_B128P2) {
    float s = tile_scale;
    if (!W2D) {                 // one 1x128 block = the whole strip
      uint32_t m = 0;
      for (int j = 0; j < TILE; j += 16) {
        uint32_t b[16];
        read16<ROWDIR>(tile, strip, j, b);
        uint32_t mm = max_abs_bits16(b);
        m = m > mm ? m : mm;
      }
      s = mx_inv_scale(mx_e8m0_from_bf16_amax(m));
    }
    if (!W2D || scale_writer)   // s = 2^(127 - c): its exponent field is 254 - c
      *(uint32_t*)out_scales32 = (254u - (__float_as_uint(s) >> 23)) * 0x01010101u;
    for (int j = 0; j < TILE; j += 16) {
      uint32_t b[16];
      read16<ROWDIR>(tile, strip, j, b);
      *(uint4*)(out_codes + j) = hw_fp8x16<F_E4M3>(b, s);
    }
  } else if (RECIPE == R_MX) {
    for (int j = 0; j < len; j += 32) {
      uint32_t b0[16], b1[16];
      read16<ROWDIR>(tile, strip, j, b0);
      read16<ROWDIR>(tile, strip, j + 16, b1);
      uint32_t m0 = max_abs_bits16(b0), m1 = max_abs_bits16(b1);
      const uint32_t c = mx_e8m0_from_bf16_amax(m0 > m1 ? m0 : m1);
      const float inv = mx_inv_scale(c);
      out_scales8[j / 32] = (uint8_t)c;
      *(uint4*)(out_codes + j) = hw_fp8x16<F_E4M3>(b0, inv);
      *(uint4*)(out_codes + j + 16) = hw_fp8x16<F_E4M3>(b1, inv);
    }
  } else if (RECIPE == R_MX4) {
    for (int j = 0; j < len; j += 32) {
      uint32_t b[32], q[32];
      float v[32];
      read16<ROWDIR>(tile, strip, j, b);
      read16<ROWDIR>(tile, strip, j + 16, b + 16);
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        v[i] = bf16_to_float(b[i]);
        const uint32_t x = b[i] & 0x7FFFu;
        m = m > x ? m : x;
      }
      const uint32_t c = mx4_e8m0_from_f32_amax(m << 16);
      const float inv = mx_inv_scale(c);
      out_scales8[j / 32] = (uint8_t)c;
      float x[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = v[i] * inv;
      if (SR) {
        uint32_t rnd[32];
        sr_strip_words<ROWDIR, 32>(a, g_row0, g_col0, j, rnd);
#pragma unroll
        for (int i = 0; i < 32; ++i) q[i] = sr_e2m1(x[i], rnd[i]);
        *(uint2*)(out_codes + j / 2) = pack_e2m1_16(q);
        *(uint2*)(out_codes + j / 2 + 8) = pack_e2m1_16(q + 16);
      } else {
        *(uint2*)(out_codes + j / 2) = make_uint2(hw_fp4x8(x), hw_fp4x8(x + 8));
        *(uint2*)(out_codes + j / 2 + 8) = make_uint2(hw_fp4x8(x + 16), hw_fp4x8(x + 24));
      }
    }
  } else {  // R_NV
    const float S = tile_scale;
    for (int j = 0; j < len; j += 16) {
      uint32_t b[16], rnd[16];
      float v[16];
      read16<ROWDIR>(tile, strip, j, b);
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = bf16_to_float(b[i]);
      if (RHT) rht16(v, rht_mask);
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        uint32_t x = __float_as_uint(v[i]) & 0x7FFFFFFFu;
        m = m > x ? m : x;
      }
      if (W2D) m = max16lanes(m);
      if (SR) sr_strip_words<ROWDIR, 16>(a, g_row0, g_col0, j, rnd);
      uint2 w;
      const uint32_t dcode = nvfp4_block<SR>(v, m, S, rnd, &w);
      *(uint2*)(out_codes + j / 2) = w;
      if (!W2D || scale_writer) out_scales8[j / 16] = (uint8_t)dcode;
    }
  }
}

template <int RECIPE, int FMT, bool ROW, bool COL, bool W2D, bool RHT, bool SR, bool AMAX>
__global__ __launch_bounds__(128) void cast_tile_kernel(CastArgs a) {
  __shared__ __align__(16) bf16_t tile[TILE * LDS_STRIDE];
  __shared__ uint32_t s_part[2];
  __shared__ uint32_t s_rht_mask;
  const int t = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.y * TILE, c0 = (int64_t)blockIdx.x * TILE;
  const int rlim = (int)min((int64_t)TILE, a.R - r0);
  const int clim = (int)min((int64_t)TILE, a.C - c0);

  // Stage the tile: 16 threads per 256-byte row, 8 rows per pass; all 16
  // loads of a thread in flight before the first LDS store (four at a time
  // left a workgroup of 128 threads with too few bytes in flight).
  uint32_t mx = 0;
  {
    const int ch = t & 15;
    uint4 vv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = (t >> 4) + 8 * i;
      vv[i] = make_uint4(0, 0, 0, 0);
      if (row < rlim && ch * 8 < clim) vv[i] = ld_nt16(a.x + (r0 + row) * a.C + c0 + ch * 8);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = (t >> 4) + 8 * i;
      const uint4 v = vv[i];
      *(uint4*)&tile[row * LDS_STRIDE + ch * 8] = v;
      if (AMAX || ((RECIPE == R_BLOCK128 || RECIPE == R_B128P2) && W2D)) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint32_t lo = w[k] & 0x7FFFu, hi = (w[k] >> 16) & 0x7FFFu;
          mx = mx > lo ? mx : lo;
          mx = mx > hi ? mx : hi;
        }
      }
    }
  }
  if (RHT && t < 64) {
    uint32_t bit = 0;
    if (t < 16) bit = philox_word0(t, 0u, 1u, 0u, (uint32_t)a.rht_seed, (uint32_t)(a.rht_seed >> 32)) & 1u;
    const uint64_t bal = __ballot(bit);
    if (t == 0) s_rht_mask = (uint32_t)bal;
  }
  if (AMAX || ((RECIPE == R_BLOCK128 || RECIPE == R_B128P2) && W2D)) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      uint32_t w = (uint32_t)__shfl_xor((int)mx, o, 64);
      mx = mx > w ? mx : w;
    }
    if ((t & 63) == 0) s_part[t >> 6] = mx;
  }
  __syncthreads();
  uint32_t tile_max_bits = 0;
  if (AMAX || ((RECIPE == R_BLOCK128 || RECIPE == R_B128P2) && W2D)) {
    tile_max_bits = s_part[0] > s_part[1] ? s_part[0] : s_part[1];
    if (AMAX && t == 0) atomicMax(a.amax_out, tile_max_bits << 16);
  }
  const uint32_t rht_mask = RHT ? s_rht_mask : 0u;

  float tile_scale = 0.0f;
  if (RECIPE == R_TENSOR || RECIPE == R_NV) tile_scale = *a.scale;
  if (RECIPE == R_BLOCK128 && W2D) tile_scale = scale_from_amax(bf16_to_float(tile_max_bits), 448.0f);
  if (RECIPE == R_B128P2 && W2D) tile_scale = mx_inv_scale(mx_e8m0_from_bf16_amax(tile_max_bits));

  if (ROW && t < rlim) {
    const int64_t gr = r0 + t;
    uint8_t* codes = (RECIPE == R_NV || RECIPE == R_MX4) ? a.row_codes + gr * (a.C / 2) + c0 / 2
                                                         : a.row_codes + gr * a.C + c0;
    uint8_t* sc8 = nullptr;
    float* sc32 = nullptr;
    bool writer = true;
    if (RECIPE == R_BLOCK128 || RECIPE == R_B128P2)
      sc32 = W2D ? (float*)a.row_scales + (r0 / 128) * (a.C / 128) + c0 / 128
                 : (float*)a.row_scales + gr * (a.C / 128) + c0 / 128;
    if ((RECIPE == R_BLOCK128 || RECIPE == R_B128P2) && W2D) writer = (t == 0);
    if (RECIPE == R_MX || RECIPE == R_MX4) sc8 = (uint8_t*)a.row_scales + gr * (a.C / 32) + c0 / 32;
    if (RECIPE == R_NV) {
      sc8 = W2D ? (uint8_t*)a.row_scales + (gr / 16) * (a.C / 16) + c0 / 16
                : (uint8_t*)a.row_scales + gr * (a.C / 16) + c0 / 16;
      if (W2D) writer = (t & 15) == 0;
    }
    quantize_strip<RECIPE, FMT, true, W2D, false, SR>(tile, t, clim, a, tile_scale, codes, sc8, sc32,
                                                      gr, c0, 0u, writer);
  }
  if (COL && t < clim) {
    const int64_t gc = c0 + t;
    uint8_t* codes = (RECIPE == R_NV || RECIPE == R_MX4) ? a.col_codes + gc * (a.R / 2) + r0 / 2
                                                         : a.col_codes + gc * a.R + r0;
    uint8_t* sc8 = nullptr;
    float* sc32 = nullptr;
    bool writer = true;
    if (RECIPE == R_BLOCK128 || RECIPE == R_B128P2)
      sc32 = W2D ? (float*)a.col_scales + (c0 / 128) * (a.R / 128) + r0 / 128
                 : (float*)a.col_scales + gc * (a.R / 128) + r0 / 128;
    if ((RECIPE == R_BLOCK128 || RECIPE == R_B128P2) && W2D) writer = (t == 0);
    if (RECIPE == R_MX || RECIPE == R_MX4) sc8 = (uint8_t*)a.col_scales + gc * (a.R / 32) + r0 / 32;
    if (RECIPE == R_NV) {
      sc8 = W2D ? (uint8_t*)a.col_scales + (gc / 16) * (a.R / 16) + r0 / 16
                : (uint8_t*)a.col_scales + gc * (a.R / 16) + r0 / 16;
      if (W2D) writer = (t & 15) == 0;
    }
    quantize_strip<RECIPE, FMT, false, W2D, RHT, SR>(tile, t, rlim, a, tile_scale, codes, sc8, sc32,
                                                     r0, gc, rht_mask, writer);
  }
}

// ---------------------------------------------------------------------------
// Single-orientation casts with 1D blocks: the common case of a cast per
// GEMM operand.  The row copy works on 8-value units (quantize_row8: a block
// of 16, 32 or 128 values is 2, 4 or 16 neighbouring lanes); the col copy
// (cast_rc_kernel below) and the Hadamard / stochastic-rounding col copy
// (cast_col_kernel) on 16-value segments of a column (quantize_segment:
// NVFP4 blocks are one segment, MX blocks two neighbouring lanes, 1x128
// blocks eight).  Block maxima reduce across lanes with DPP moves.
//
// Encoding uses the gfx950 conversion instructions, clamped first so that
// they saturate (see hw_fp8x4 / hw_fp4x8 above).
// ---------------------------------------------------------------------------
// Max of the 15-bit magnitudes of 16 bf16 values held as 8 packed words.
__device__ __forceinline__ uint32_t bf16_absmax16(const uint32_t* w) {
  u16x2 m = {0, 0};
#pragma unroll
  for (int i = 0; i < 8; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
  return m.x > m.y ? m.x : m.y;
}

__device__ __forceinline__ void bf16x16_to_f32(const uint32_t* w, float* v) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// Quantize one segment.  v: 16 fp32 values; mbits: max |value| bits over the
// segment (fp32 bits); the group (block) reduction happens here.  Writes the
// codes to `codes` (16 bytes for FP8, 8 for E2M1) and, from the lane that
// owns the block's first segment, the block scale.
//  RECIPE R_TENSOR: s = tensor scale; R_MX: 2-lane blocks; R_BLOCK128:
//  8-lane blocks; R_NV: one-segment blocks with encode scale S = tscale;
//  R_MX4: 2-lane blocks, E2M1 codes.
template <int RECIPE, int FMT, bool SR>
__device__ __forceinline__ void quantize_segment(const float* v, uint32_t mbits, float tscale, bool valid,
                                                 uint8_t* codes, uint8_t* sc8, float* sc32, bool writer,
                                                 const uint32_t* rnd) {
  if (RECIPE == R_TENSOR || RECIPE == R_MX || RECIPE == R_BLOCK128 || RECIPE == R_B128P2) {
    float s = tscale;
    if (RECIPE == R_MX) {
      const uint32_t m = group_max<2>(mbits);
      // the E8M0 rule works on the bf16 bits of the block maximum
      const uint32_t c = mx_e8m0_from_bf16_amax(m >> 16);
      s = mx_inv_scale(c);
      if (valid && writer) *sc8 = (uint8_t)c;
    } else if (RECIPE == R_BLOCK128) {
      const uint32_t m = group_max<8>(mbits);
      s = scale_from_amax(__uint_as_float(m), 448.0f);
      if (valid && writer) *sc32 = 1.0f / s;
    } else if (RECIPE == R_B128P2) {
      const uint32_t c = mx_e8m0_from_bf16_amax(group_max<8>(mbits) >> 16);
      s = mx_inv_scale(c);
      if (valid && writer) *(uint32_t*)sc32 = c * 0x01010101u;
    }
    uint4 o;
    o.x = hw_fp8x4<FMT>(v[0] * s, v[1] * s, v[2] * s, v[3] * s);
    o.y = hw_fp8x4<FMT>(v[4] * s, v[5] * s, v[6] * s, v[7] * s);
    o.z = hw_fp8x4<FMT>(v[8] * s, v[9] * s, v[10] * s, v[11] * s);
    o.w = hw_fp8x4<FMT>(v[12] * s, v[13] * s, v[14] * s, v[15] * s);
    if (valid) *(uint4*)codes = o;
  } else if (RECIPE == R_MX4) {
    const uint32_t c = mx4_e8m0_from_f32_amax(group_max<2>(mbits));
    const float s = mx_inv_scale(c);
    if (valid && writer) *sc8 = (uint8_t)c;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = v[i] * s;
    uint2 o;
    if (SR) {
      uint32_t q[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) q[i] = sr_e2m1(x[i], rnd[i]);
      o = pack_e2m1_16(q);
    } else {
      o.x = hw_fp4x8(x);
      o.y = hw_fp4x8(x + 8);
    }
    if (valid) *(uint2*)codes = o;
  } else {  // R_NV
    uint2 o;
    const uint32_t d_code = nvfp4_block<SR>(v, mbits, tscale, rnd, &o);
    if (valid) {
      *(uint2*)codes = o;
      *sc8 = (uint8_t)d_code;
    }
  }
}

// Fold a per-thread |x| maximum (fp32 bits) into *out: wave reduction, one
// value per workgroup through LDS, then one atomic from thread 0 only when
// the workgroup maximum exceeds what *out already holds (the running maximum
// settles early, so most workgroups skip the atomic).
__device__ __forceinline__ void wg_amax_fold(uint32_t v, uint32_t* out, uint32_t* s_part) {
  v = group_max<64>(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) s_part[w] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = s_part[0];
    for (int i = 1; i < (int)(blockDim.x >> 6); ++i) m = m > s_part[i] ? m : s_part[i];
    const uint32_t cur = __builtin_nontemporal_load(out);
    if (m > cur) atomicMax(out, m);
  }
}

// Quantize 8 row values v (fp32) held by a lane, with the row block spread
// over 2 (NVFP4), 4 (MX) or 16 (1x128) neighbouring lanes (ch: the lane's
// place among 16 such lanes); writes the codes (8 bytes, or 4 for E2M1) and,
// from the block's first lane, its scale.  SR (E2M1 recipes): rnd holds the
// values' stochastic-rounding words.
template <int RECIPE, int FMT, bool SR = false>
__device__ __forceinline__ void quantize_row8(const float* v, uint32_t mbits, float tscale, bool valid, int ch,
                                              uint8_t* codes, uint8_t* sc8, float* sc32,
                                              const uint32_t* rnd = nullptr) {
  auto e2m1x8 = [&](const float* x) {
    if (!SR) return hw_fp4x8(x);
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= sr_e2m1(x[i], rnd[i]) << (4 * i);
    return w;
  };
  if (RECIPE == R_NV || RECIPE == R_MX4) {
    uint32_t w;
    bool writer;
    uint32_t scode;
    if (RECIPE == R_NV) {
      const uint32_t m = group_max<2>(mbits);
      const float S = tscale;
      const NvScale4 sc = nv_block_scale((__uint_as_float(m) / 6.0f) * S, S);
      scode = sc.code;
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = v[i] * sc.e_b;
      w = e2m1x8(x);
      writer = (ch & 1) == 0;
    } else {
      scode = mx4_e8m0_from_f32_amax(group_max<4>(mbits));
      const float s = mx_inv_scale(scode);
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = v[i] * s;
      w = e2m1x8(x);
      writer = (ch & 3) == 0;
    }
    if (valid) {
      *(uint32_t*)codes = w;
      if (writer) *sc8 = (uint8_t)scode;
    }
    return;
  }
  float s = tscale;
  bool writer = false;
  uint32_t word = 0;
  if (RECIPE == R_MX) {
    const uint32_t c = mx_e8m0_from_bf16_amax(group_max<4>(mbits) >> 16);
    s = mx_inv_scale(c);
    writer = (ch & 3) == 0;
    word = c;
  } else if (RECIPE == R_BLOCK128) {
    s = scale_from_amax(__uint_as_float(group_max<16>(mbits)), 448.0f);
    writer = ch == 0;
  } else if (RECIPE == R_B128P2) {
    const uint32_t c = mx_e8m0_from_bf16_amax(group_max<16>(mbits) >> 16);
    s = mx_inv_scale(c);
    writer = ch == 0;
    word = c * 0x01010101u;
  }
  uint2 o;
  o.x = hw_fp8x4<FMT>(v[0] * s, v[1] * s, v[2] * s, v[3] * s);
  o.y = hw_fp8x4<FMT>(v[4] * s, v[5] * s, v[6] * s, v[7] * s);
  if (valid) {
    *(uint2*)codes = o;
    if (writer) {
      if (RECIPE == R_MX) *sc8 = (uint8_t)word;
      else if (RECIPE == R_BLOCK128) *sc32 = 1.0f / s;
      else if (RECIPE == R_B128P2) *(uint32_t*)sc32 = word;
    }
  }
}

// Row copy: a lane quantizes units of 8 consecutive values (one 16-byte
// load), U = 8 units per step; unit q of the flat tensor is values 8 q ..
// 8 q + 7, and the 64 lanes of one load instruction take 64 consecutive
// units, so every load reads 1 KB of contiguous input (32 bytes per lane as
// two 16-byte loads, every instruction touching 2 KB, streamed 6% slower).
// Every output is row-major with the blocks along the row and the row
// length is a multiple of the block, so input, codes, block scales and the
// SR counter are all linear in q, a block of 16, 32 or 128 values is 2, 4 or
// 16 neighbouring lanes (never straddling a row), and a block is either
// wholly inside the tensor or wholly past its end.  No LDS.
template <int RECIPE, int FMT, bool SR, bool AMAX>
__global__ __launch_bounds__(256) void cast_row_kernel(CastArgs a, int64_t nseg) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * 4;
  const int64_t wave0 = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  float tscale = 0.0f;
  if (RECIPE == R_TENSOR || RECIPE == R_NV) tscale = *a.scale;
  constexpr bool E2M1 = RECIPE == R_NV || RECIPE == R_MX4;
  const int64_t nu = 2 * nseg;
  uint32_t amx = 0;
  constexpr int U = 8;
  for (int64_t wt = wave0; wt * 64 * U < nu; wt += waves) {
    uint4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t q = wt * 64 * U + u * 64 + lane;
      w[u] = ld_nt16(a.x + (q < nu ? q : 0) * 8);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t q = wt * 64 * U + u * 64 + lane;
      const bool valid = q < nu;
      const uint32_t w4[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
      u16x2 m2 = {0, 0};
#pragma unroll
      for (int k = 0; k < 4; ++k) m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, w4[k] & 0x7FFF7FFFu));
      const uint32_t m8 = m2.x > m2.y ? m2.x : m2.y;
      if (AMAX && valid) amx = amx > m8 ? amx : m8;
      float f[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        f[2 * k] = __uint_as_float(w4[k] << 16);
        f[2 * k + 1] = __uint_as_float(w4[k] & 0xFFFF0000u);
      }
      uint32_t rnd[8];
      if (SR) {                                   // logical indices 8 q .. 8 q + 7: two calls
        const uint4 r0 = sr_words4((uint64_t)(2 * q), a.seed), r1 = sr_words4((uint64_t)(2 * q + 1), a.seed);
        rnd[0] = r0.x; rnd[1] = r0.y; rnd[2] = r0.z; rnd[3] = r0.w;
        rnd[4] = r1.x; rnd[5] = r1.y; rnd[6] = r1.z; rnd[7] = r1.w;
      }
      uint8_t* codes = a.row_codes + q * (E2M1 ? 4 : 8);
      uint8_t* sc8 = nullptr;
      float* sc32 = nullptr;
      if (RECIPE == R_MX || RECIPE == R_MX4) sc8 = (uint8_t*)a.row_scales + q / 4;
      else if (RECIPE == R_NV) sc8 = (uint8_t*)a.row_scales + q / 2;
      else if (RECIPE == R_BLOCK128 || RECIPE == R_B128P2) sc32 = (float*)a.row_scales + q / 16;
      quantize_row8<RECIPE, FMT, SR>(f, m8 << 16, tscale, valid, lane & 15, codes, sc8, sc32, rnd);
    }
  }
  if (AMAX) {
    __shared__ uint32_t s_part[4];
    wg_amax_fold(amx << 16, a.amax_out, s_part);
  }
}

// Col copy (the transposed tensor, blocks along x's rows).  A workgroup
// stages a 256-row x 64-column tile of x in LDS; thread t takes rows
// 16 (t % 16) .. + 15 of the 4 columns 4 (t / 16) .. + 3, so each of its 4
// segments is 16 consecutive rows of one column, i.e. 16 consecutive values
// of an output row.  LDS: row pitch 136 B (34 dwords: rows 16 apart land in
// opposite bank halves) and the 8-byte column group g of row r stored at
// g ^ ((r >> 4) & 14): the 64-lane 8-byte column reads are conflict-free.
constexpr int CT_R = 256, CT_C = 64, CT_PITCH = 136;

template <int RECIPE, int FMT, bool RHT, bool SR, bool AMAX>
__global__ __launch_bounds__(256, 2) void cast_col_kernel(CastArgs a) {
  __shared__ __align__(16) uint8_t tile[CT_R * CT_PITCH];
  // MXFP4 with stochastic rounding: the random words of columns 2 and 3 wait
  // in LDS (word j of thread t at j * 256 + t, each thread its own slots)
  // instead of 32 registers, which kept that variant from spilling
  constexpr bool WORDS_LDS = SR && RECIPE == R_MX4;
  __shared__ uint32_t wlds[WORDS_LDS ? 32 * 256 : 1];
  const int t = threadIdx.x, lane = t & 63;
  uint32_t rht_mask = 0;
  if (RHT) {
    // bit j of the mask from lane j (Philox counter (j, 0, 1, 0), bit 0 of word 0)
    const uint32_t bit = lane < 16 ? (philox_word0((uint32_t)lane, 0u, 1u, 0u, (uint32_t)a.rht_seed,
                                                   (uint32_t)(a.rht_seed >> 32)) & 1u) : 0u;
    rht_mask = (uint32_t)__ballot(bit);
  }
  float tscale = 0.0f;
  if (RECIPE == R_TENSOR || RECIPE == R_NV) tscale = *a.scale;
  // Tiles in row-major order of the (rows / 256) x (cols / 64) tile grid.
  // A launch with one workgroup per tile gives each its own tile; the fused-
  // amax launch is shorter, and each workgroup walks tiles tile,
  // tile + gridDim.x, ... so that only that many same-address atomics end it.
  const int64_t gx = (a.C + CT_C - 1) / CT_C;
  const int64_t ntiles = gx * ((a.R + CT_R - 1) / CT_R);
  uint32_t amx = 0;
  for (int64_t tl = (int64_t)blockIdx.y * gridDim.x + blockIdx.x; tl < ntiles;
       tl += (int64_t)gridDim.x * gridDim.y) {
    const int64_t r0 = (tl / gx) * CT_R, c0 = (tl % gx) * CT_C;
    const int rlim = (int)min((int64_t)CT_R, a.R - r0);
    const int clim = (int)min((int64_t)CT_C, a.C - c0);
    // fill: 8 lanes per 128-byte row segment, 32 rows per pass, 8 passes
    {
      const int ch = t & 7;
      uint4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = (t >> 3) + 32 * i;
        v[i] = make_uint4(0, 0, 0, 0);
        if (row < rlim && ch * 8 < clim) v[i] = ld_nt16(a.x + (r0 + row) * a.C + c0 + ch * 8);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = (t >> 3) + 32 * i;
        const int g = (2 * ch) ^ ((row >> 4) & 14);
        // odd rows start 8 bytes into a 16-byte line: two 8-byte stores
        *(uint2*)(tile + row * CT_PITCH + g * 8) = make_uint2(v[i].x, v[i].y);
        *(uint2*)(tile + row * CT_PITCH + g * 8 + 8) = make_uint2(v[i].z, v[i].w);
      }
    }
    __syncthreads();

    const int rs = t & 15, cg = t >> 4;
    // 16 rows x 4 columns: wv[i] = 4 bf16 of row 16 rs + i
    uint2 wv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 16 * rs + i;
      const int g = cg ^ ((row >> 4) & 14);
      wv[i] = *(const uint2*)(tile + row * CT_PITCH + g * 8);
    }
    // stochastic rounding: the thread's 4 columns 4 cg .. 4 cg + 3 are one
    // aligned group of a row of x, so one call per row serves all four
    // (one call in flight at a time: hoisting all sixteen multiplies the live
    // registers, and occupancy hides the chain's latency better)
    uint32_t rndc[WORDS_LDS ? 2 : 4][16];
    if (SR) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint64_t idx = (uint64_t)((r0 + 16 * rs + i) * a.C + c0 + 4 * cg);
        const uint4 r4 = sr_words4(idx >> 2, a.seed);
        rndc[0][i] = r4.x;
        rndc[1][i] = r4.y;
        if constexpr (WORDS_LDS) {
          wlds[i * 256 + t] = r4.z;
          wlds[(16 + i) * 256 + t] = r4.w;
        } else {
          rndc[WORDS_LDS ? 0 : 2][i] = r4.z;
          rndc[WORDS_LDS ? 1 : 3][i] = r4.w;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t word = (c < 2) ? wv[i].x : wv[i].y;
        v[i] = __uint_as_float((c & 1) ? (word & 0xFFFF0000u) : (word << 16));
      }
      const int col = 4 * cg + c;
      const bool valid = (16 * rs < rlim) && (col < clim);
      uint32_t mbits = 0;
      if (RHT) {
        rht16(v, rht_mask);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t x = __float_as_uint(v[i]) & 0x7FFFFFFFu;
          mbits = mbits > x ? mbits : x;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t x = __float_as_uint(v[i]) & 0x7FFFFFFFu;
          mbits = mbits > x ? mbits : x;
        }
      }
      if (AMAX && valid) amx = amx > mbits ? amx : mbits;
      const int64_t gc = c0 + col, gr = r0 + 16 * rs;
      if (RECIPE == R_CHAN)   // the column's amax (fp32 bits), measured by chan_colmax_kernel
        tscale = scale_from_amax(__uint_as_float(((const uint32_t*)a.col_scales)[valid ? gc : c0]), 448.0f);
      uint8_t* codes = (RECIPE == R_NV || RECIPE == R_MX4) ? a.col_codes + gc * (a.R / 2) + gr / 2
                                                           : a.col_codes + gc * a.R + gr;
      uint8_t* sc8 = nullptr;
      float* sc32 = nullptr;
      bool writer = true;
      if (RECIPE == R_MX || RECIPE == R_MX4) {
        sc8 = (uint8_t*)a.col_scales + gc * (a.R / 32) + gr / 32;
        writer = (rs & 1) == 0;
      } else if (RECIPE == R_NV) {
        sc8 = (uint8_t*)a.col_scales + gc * (a.R / 16) + gr / 16;
      } else if (RECIPE == R_BLOCK128 || RECIPE == R_B128P2) {
        sc32 = (float*)a.col_scales + gc * (a.R / 128) + gr / 128;
        writer = (rs & 7) == 0;
      }
      uint32_t rl[16];
      const uint32_t* rnd = rndc[c & (WORDS_LDS ? 1 : 3)];
      if (WORDS_LDS && c >= 2) {
#pragma unroll
        for (int i = 0; i < 16; ++i) rl[i] = wlds[((c - 2) * 16 + i) * 256 + t];
        rnd = rl;
      }
      quantize_segment<RECIPE == R_CHAN ? R_TENSOR : RECIPE, FMT, SR>(v, mbits, tscale, valid, codes, sc8, sc32,
                                                                       writer, rnd);
      if (SR) __builtin_amdgcn_sched_barrier(0);   // one column at a time: the words already hold 64 registers
    }
    __syncthreads();   // every read of this tile is done before the next fill
  }
  if (AMAX) {
    __shared__ uint32_t s_part[4];
    wg_amax_fold(amx, a.amax_out, s_part);
  }
}

// ---------------------------------------------------------------------------
// Col copy, alone or with the row copy from the same read, for 1D blocks
// without the Hadamard transform or stochastic rounding.  A workgroup
// stages a 256-row x 128-column tile of x in LDS (two 64-column halves laid
// out as cast_col_kernel's tile, so the column reads stay conflict-free);
// every row of the tile is read as one 256-byte piece (a read probe of this
// pattern streams faster than 128-byte pieces).  Fill: lane ch = t % 16
// holds 8 values of columns 8 ch .. 8 ch + 7 of rows t / 16 + 16 i; with
// ROW it quantizes them on the spot -- the lanes of one row piece are 16
// neighbouring lanes, so a block of 16, 32 or 128 values is 2, 4 or 16 lanes
// -- and stores the row copy's codes (16 lanes write 128 contiguous bytes).
// Then the col copy as in cast_col_kernel, once per half.
// ---------------------------------------------------------------------------
// The 256 x 128 tile (two halves) with a grid of at most 1024 workgroups:
// 64-column tiles made the two-copy cast 35% slower (8 lanes per 128-byte
// row piece of the row copy), 512 or 2048 workgroups no faster.
constexpr int RC_NH = 2;
constexpr int RC_GRID = 1024;

template <int RECIPE, int FMT, bool ROW, bool AMAX, int NH>
__global__ __launch_bounds__(256) void cast_rc_kernel(CastArgs a) {
  static_assert(NH == 1 || NH == 2, "one or two 64-column halves");
  constexpr int TC = 64 * NH;               // tile columns
  constexpr int LPR = 8 * NH;               // lanes per row piece
  constexpr int RPP = 256 / LPR;            // rows per fill pass
  constexpr int NP = CT_R / RPP;            // fill passes (loads per lane)
  __shared__ __align__(16) uint8_t tile[NH * CT_R * CT_PITCH];
  const int t = threadIdx.x;
  float tscale = 0.0f;
  if (RECIPE == R_TENSOR || RECIPE == R_NV) tscale = *a.scale;
  constexpr bool E2M1 = RECIPE == R_NV || RECIPE == R_MX4;
  const int64_t gx = (a.C + TC - 1) / TC;
  const int64_t ntiles = gx * ((a.R + CT_R - 1) / CT_R);
  const int ch = t % LPR;
  const int half = ch >> 3, c8 = ch & 7;
  uint32_t amx = 0;
  // The workgroup walks tiles tl, tl + gridDim.x, ...; the loads of the next
  // tile are issued before the col phase of the current one, so they are in
  // flight while it computes.
  uint4 v[NP];
  auto issue = [&](int64_t tl) {
    const int64_t r0 = (tl / gx) * CT_R, c0 = (tl % gx) * TC;
    const int rlim = (int)min((int64_t)CT_R, a.R - r0);
    const bool cvalid = ch * 8 < (int)min((int64_t)TC, a.C - c0);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int row = t / LPR + RPP * i;
      v[i] = make_uint4(0, 0, 0, 0);
      if (row < rlim && cvalid) v[i] = ld_nt16(a.x + (r0 + row) * a.C + c0 + ch * 8);
    }
  };
  if ((int64_t)blockIdx.x < ntiles) issue(blockIdx.x);
  for (int64_t tl = blockIdx.x; tl < ntiles; tl += gridDim.x) {
    const int64_t r0 = (tl / gx) * CT_R, c0 = (tl % gx) * TC;
    const int rlim = (int)min((int64_t)CT_R, a.R - r0);
    const int clim = (int)min((int64_t)TC, a.C - c0);
    // fill: LPR lanes per row piece (8 values each), RPP rows per pass
    {
      const bool cvalid = ch * 8 < clim;
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int row = t / LPR + RPP * i;
        uint8_t* th = tile + half * (CT_R * CT_PITCH);
        const int g = (2 * c8) ^ ((row >> 4) & 14);
        *(uint2*)(th + row * CT_PITCH + g * 8) = make_uint2(v[i].x, v[i].y);
        *(uint2*)(th + row * CT_PITCH + g * 8 + 8) = make_uint2(v[i].z, v[i].w);
        const uint32_t w4[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        u16x2 m2 = {0, 0};
#pragma unroll
        for (int k = 0; k < 4; ++k) m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, w4[k] & 0x7FFF7FFFu));
        const uint32_t m16 = m2.x > m2.y ? m2.x : m2.y;
        if (AMAX) amx = amx > m16 ? amx : m16;
        if (ROW) {
          float f[8];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            f[2 * k] = __uint_as_float(w4[k] << 16);
            f[2 * k + 1] = __uint_as_float(w4[k] & 0xFFFF0000u);
          }
          const bool valid = row < rlim && cvalid;
          const int64_t gr = r0 + row, gcol = c0 + ch * 8;
          uint8_t* codes = E2M1 ? a.row_codes + gr * (a.C / 2) + gcol / 2 : a.row_codes + gr * a.C + gcol;
          uint8_t* sc8 = nullptr;
          float* sc32 = nullptr;
          if (RECIPE == R_MX || RECIPE == R_MX4) sc8 = (uint8_t*)a.row_scales + gr * (a.C / 32) + gcol / 32;
          if (RECIPE == R_NV) sc8 = (uint8_t*)a.row_scales + gr * (a.C / 16) + gcol / 16;
          if (RECIPE == R_BLOCK128 || RECIPE == R_B128P2) sc32 = (float*)a.row_scales + gr * (a.C / 128) + gcol / 128;
          quantize_row8<RECIPE, FMT>(f, m16 << 16, tscale, valid, ch, codes, sc8, sc32);
        }
      }
    }
    // the tile's LDS writes are visible to every wave (the global stores of
    // the row copy need not have landed)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (tl + (int64_t)gridDim.x < ntiles) issue(tl + gridDim.x);

    // col copy: thread t takes rows 16 (t % 16) .. + 15 of 4 columns of each half
    const int rs = t & 15, cg = t >> 4;
#pragma unroll
    for (int half = 0; half < NH; ++half) {
      const uint8_t* th = tile + half * (CT_R * CT_PITCH);
      uint2 wv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 16 * rs + i;
        const int g = cg ^ ((row >> 4) & 14);
        wv[i] = *(const uint2*)(th + row * CT_PITCH + g * 8);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float cv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t word = (c < 2) ? wv[i].x : wv[i].y;
          cv[i] = __uint_as_float((c & 1) ? (word & 0xFFFF0000u) : (word << 16));
        }
        const int col = 64 * half + 4 * cg + c;
        const bool valid = (16 * rs < rlim) && (col < clim);
        uint32_t mbits = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t x = __float_as_uint(cv[i]) & 0x7FFFFFFFu;
          mbits = mbits > x ? mbits : x;
        }
        const int64_t gc = c0 + col, gr = r0 + 16 * rs;
        uint8_t* codes = E2M1 ? a.col_codes + gc * (a.R / 2) + gr / 2 : a.col_codes + gc * a.R + gr;
        uint8_t* sc8 = nullptr;
        float* sc32 = nullptr;
        bool writer = true;
        if (RECIPE == R_MX || RECIPE == R_MX4) {
          sc8 = (uint8_t*)a.col_scales + gc * (a.R / 32) + gr / 32;
          writer = (rs & 1) == 0;
        } else if (RECIPE == R_NV) {
          sc8 = (uint8_t*)a.col_scales + gc * (a.R / 16) + gr / 16;
        } else if (RECIPE == R_BLOCK128 || RECIPE == R_B128P2) {
          sc32 = (float*)a.col_scales + gc * (a.R / 128) + gr / 128;
          writer = (rs & 7) == 0;
        }
        quantize_segment<RECIPE, FMT, false>(cv, mbits, tscale, valid, codes, sc8, sc32, writer, nullptr);
      }
    }
    // every LDS read of this tile is done before the next fill
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
  if (AMAX) {
    __shared__ uint32_t s_part[4];
    wg_amax_fold(amx << 16, a.amax_out, s_part);
  }
}

// ---------------------------------------------------------------------------
// Channel-wise FP8: one scale per row of the copy.
//
// Row copy: a team of T lanes (one wave, or the whole 256-thread workgroup
// for long rows) owns a row; lane l holds the row's 8-value units l, l + T,
// ... (up to 2 NCH of them, one 16-byte load each) in registers, so the row
// is read from HBM once: max over the team, scale, encode, store.  Rows
// longer than 256 * 16 * 16 values (NCH = 0) are read twice (the second
// read mostly from L2).
//
// Col copy: one scale per column of x.  chan_colmax_kernel folds column
// maxima into col_scales (fp32 bits, cleared first); cast_col_kernel
// <R_CHAN> encodes with them; chan_finalize_kernel turns each maximum into
// the stored fp32(1 / s) in place.
// ---------------------------------------------------------------------------
template <int T, int NCH>
__global__ __launch_bounds__(256) void chan_row_kernel(CastArgs a) {
  constexpr int TEAMS = 256 / T;
  const int tl = threadIdx.x % T;
  const int64_t row = (int64_t)blockIdx.x * TEAMS + threadIdx.x / T;
  const bool live = row < a.R;
  const int64_t spr = a.C / 16;
  const bf16_t* xr = a.x + (live ? row : 0) * a.C;
  uint8_t* cr = a.row_codes + (live ? row : 0) * a.C;
  __shared__ uint32_t s_part[4];
  uint32_t m = 0;
  if (NCH > 0) {
    // 8-value units j T + tl of the row (one 16-byte load each, so the
    // lanes of a load instruction read contiguous input)
    const int64_t upr = 2 * spr;
    uint4 w[NCH > 0 ? 2 * NCH : 1];
#pragma unroll
    for (int j = 0; j < 2 * NCH; ++j) {
      const int64_t q = (int64_t)j * T + tl;
      w[j] = (live && q < upr) ? ld_nt16(xr + q * 8) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int j = 0; j < 2 * NCH; ++j) {
      const uint32_t mj = bf16_absmax8(w[j]);
      m = m > mj ? m : mj;
    }
    m = group_max<64>(m);
    if (T == 256) {
      if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = m;
      __syncthreads();
      m = s_part[0];
#pragma unroll
      for (int i = 1; i < 4; ++i) m = m > s_part[i] ? m : s_part[i];
    }
    const float s = scale_from_amax(__uint_as_float(m << 16), 448.0f);
#pragma unroll
    for (int j = 0; j < 2 * NCH; ++j) {
      const int64_t q = (int64_t)j * T + tl;
      float f[8];
      bf16x8_to_f32(w[j], f);
      quantize_row8<R_TENSOR, F_E4M3>(f, 0u, s, live && q < upr, 0, cr + q * 8, nullptr, nullptr);
    }
    if (live && tl == 0) ((float*)a.row_scales)[row] = 1.0f / s;
  } else {
    for (int64_t sg = tl; sg < spr; sg += T) {
      uint32_t w[8];
      const uint4 v0 = ld_nt16(xr + sg * 16), v1 = ld_nt16(xr + sg * 16 + 8);
      w[0] = v0.x; w[1] = v0.y; w[2] = v0.z; w[3] = v0.w;
      w[4] = v1.x; w[5] = v1.y; w[6] = v1.z; w[7] = v1.w;
      const uint32_t mj = bf16_absmax16(w);
      m = m > mj ? m : mj;
    }
    m = group_max<64>(m);
    if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = m;
    __syncthreads();
    m = s_part[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) m = m > s_part[i] ? m : s_part[i];
    const float s = scale_from_amax(__uint_as_float(m << 16), 448.0f);
    for (int64_t sg = tl; sg < spr; sg += T) {
      uint32_t w[8];
      const uint4 v0 = *(const uint4*)(xr + sg * 16), v1 = *(const uint4*)(xr + sg * 16 + 8);
      w[0] = v0.x; w[1] = v0.y; w[2] = v0.z; w[3] = v0.w;
      w[4] = v1.x; w[5] = v1.y; w[6] = v1.z; w[7] = v1.w;
      float v[16];
      bf16x16_to_f32(w, v);
      quantize_segment<R_TENSOR, F_E4M3, false>(v, 0u, s, true, cr + sg * 16, nullptr, nullptr, false, nullptr);
    }
    if (tl == 0) ((float*)a.row_scales)[row] = 1.0f / s;
  }
}

// Column maxima of x: lane l of a wave reads columns c0 + 8 l .. + 7 of one
// row at a time (a wave covers 512 columns of a row, 1 KB contiguous); the
// four waves take rows 4 apart in a chunk of `rows_per_wg` rows.  The
// workgroup's 512 maxima then go to col_scales (fp32 bits of |x|) with one
// atomic max each, skipped when the stored value is already as large.
constexpr int CM_COLS = 512;

__global__ __launch_bounds__(256) void chan_colmax_kernel(CastArgs a, int rows_per_wg) {
  __shared__ uint32_t part[4][CM_COLS];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t c = (int64_t)blockIdx.x * CM_COLS + 8 * lane;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_wg;
  const int64_t r1 = min(a.R, r0 + rows_per_wg);
  u16x2 m[4] = {{0, 0}, {0, 0}, {0, 0}, {0, 0}};
  if (c < a.C) {
    int64_t r = r0 + w;
    for (; r + 12 < r1; r += 16) {          // four rows per step, loads first
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = ld_nt16(a.x + (r + 4 * u) * a.C + c);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        m[0] = __builtin_elementwise_max(m[0], __builtin_bit_cast(u16x2, v[u].x & 0x7FFF7FFFu));
        m[1] = __builtin_elementwise_max(m[1], __builtin_bit_cast(u16x2, v[u].y & 0x7FFF7FFFu));
        m[2] = __builtin_elementwise_max(m[2], __builtin_bit_cast(u16x2, v[u].z & 0x7FFF7FFFu));
        m[3] = __builtin_elementwise_max(m[3], __builtin_bit_cast(u16x2, v[u].w & 0x7FFF7FFFu));
      }
    }
    for (; r < r1; r += 4) {
      const uint4 v = ld_nt16(a.x + r * a.C + c);
      m[0] = __builtin_elementwise_max(m[0], __builtin_bit_cast(u16x2, v.x & 0x7FFF7FFFu));
      m[1] = __builtin_elementwise_max(m[1], __builtin_bit_cast(u16x2, v.y & 0x7FFF7FFFu));
      m[2] = __builtin_elementwise_max(m[2], __builtin_bit_cast(u16x2, v.z & 0x7FFF7FFFu));
      m[3] = __builtin_elementwise_max(m[3], __builtin_bit_cast(u16x2, v.w & 0x7FFF7FFFu));
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    part[w][8 * lane + 2 * i] = m[i].x;
    part[w][8 * lane + 2 * i + 1] = m[i].y;
  }
  __syncthreads();
  uint32_t* amax = (uint32_t*)a.col_scales;
  for (int i = threadIdx.x; i < CM_COLS; i += 256) {
    const int64_t col = (int64_t)blockIdx.x * CM_COLS + i;
    if (col >= a.C) break;
    uint32_t v = part[0][i];
#pragma unroll
    for (int k = 1; k < 4; ++k) v = v > part[k][i] ? v : part[k][i];
    v <<= 16;                                // fp32 bits of the bf16 maximum
    if (v > __builtin_nontemporal_load(amax + col)) atomicMax(amax + col, v);
  }
}

__global__ void chan_finalize_kernel(float* sc, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) sc[i] = 1.0f / scale_from_amax(sc[i], 448.0f);
}

__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

template <int T, int NCH>
static void launch_chan_row(const CastArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((chan_row_kernel<T, NCH>), dim3((unsigned)ceil_div(a.R, 256 / T)), dim3(256), 0, stream, a);
}

// The channel-wise cast: row copy, then col copy.
static pbs_status cast_channel(const CastArgs& a, bool row, bool col, hipStream_t stream) {
  if (row && a.R > 0) {
    if (a.C == 0) {   // empty rows: scale 1
      hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)std::min<int64_t>(ceil_div(a.R, 256), 1024)), dim3(256), 0,
                         stream, (uint32_t*)a.row_scales, a.R, 0x3F800000u);
    } else {
      const int64_t spr = a.C / 16;
      log_dispatch("cast_channel_row rows=%lld cols=%lld", (long long)a.R, (long long)a.C);
      if (spr <= 64) launch_chan_row<64, 1>(a, stream);
      else if (spr <= 128) launch_chan_row<64, 2>(a, stream);
      else if (spr <= 256) launch_chan_row<64, 4>(a, stream);
      else if (spr <= 512) launch_chan_row<64, 8>(a, stream);
      else if (spr <= 1024) launch_chan_row<256, 4>(a, stream);
      else if (spr <= 2048) launch_chan_row<256, 8>(a, stream);
      else if (spr <= 4096) launch_chan_row<256, 16>(a, stream);
      else launch_chan_row<256, 0>(a, stream);
    }
  }
  if (col && a.C > 0) {
    if (a.R == 0) {
      hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)std::min<int64_t>(ceil_div(a.C, 256), 1024)), dim3(256), 0,
                         stream, (uint32_t*)a.col_scales, a.C, 0x3F800000u);
    } else {
      hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)std::min<int64_t>(ceil_div(a.C, 256), 1024)), dim3(256), 0,
                         stream, (uint32_t*)a.col_scales, a.C, 0u);
      // about 2048 workgroups, chunks of whole 16-row steps
      const int64_t gx = ceil_div(a.C, CM_COLS);
      int64_t rpw = ceil_div(a.R * gx, 2048);
      rpw = std::max<int64_t>(16, ceil_div(rpw, 16) * 16);
      const dim3 g1((unsigned)gx, (unsigned)ceil_div(a.R, rpw));
      log_dispatch("cast_channel_col rows=%lld cols=%lld colmax grid=%ux%u", (long long)a.R, (long long)a.C, g1.x,
                   g1.y);
      hipLaunchKernelGGL(chan_colmax_kernel, g1, dim3(256), 0, stream, a, (int)rpw);
      const dim3 g2((unsigned)(ceil_div(a.C, CT_C) * ceil_div(a.R, CT_R)), 1);
      hipLaunchKernelGGL((cast_col_kernel<R_CHAN, F_E4M3, false, false, false>), g2, dim3(256), 0, stream, a);
      hipLaunchKernelGGL(chan_finalize_kernel, dim3((unsigned)ceil_div(a.C, 256)), dim3(256), 0, stream,
                         (float*)a.col_scales, a.C);
    }
  }
  return check_launch("pbs_cast");
}

__global__ void zero_u32_kernel(uint32_t* p) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *p = 0u;
}

typedef void (*cast_fn)(CastArgs);

typedef void (*cast_row_fn)(CastArgs, int64_t);

// Kernel choice: single-orientation casts with 1D blocks take the row / col
// kernels; 2D weight blocks and two-copy casts take the tile kernel.
struct CastPick {
  cast_fn tile = nullptr, col = nullptr, rc = nullptr;
  cast_row_fn row = nullptr;
  int rc_cols = 0;                          // tile width of the row+col kernel
};

// 1D blocks: the row kernel for a row copy; the 256 x 128 row+col kernel for
// a plain col copy and for both copies from one read; the 256 x 64 col
// kernel for col copies with the Hadamard transform or stochastic rounding;
// the 128 x 128 tile kernel for 2D blocks and two stochastically rounded
// copies.
template <int RECIPE, int FMT, bool W2D, bool RHT, bool SR, bool AMAX>
static CastPick pick_orient(int mask) {
  CastPick p;
  if (!W2D && mask == PBS_ROW && !RHT) p.row = cast_row_kernel<RECIPE, FMT, SR, AMAX>;
  else if (!W2D && !RHT && !SR && mask == PBS_COL) {
    p.rc = cast_rc_kernel<RECIPE, FMT, false, AMAX, RC_NH>;
    p.rc_cols = 64 * RC_NH;
  } else if (!W2D && !RHT && !SR && mask == (PBS_ROW | PBS_COL)) {   // a 1x128 row block needs 128 columns
    constexpr int nh = (RECIPE == R_BLOCK128 || RECIPE == R_B128P2) ? 2 : RC_NH;
    p.rc = cast_rc_kernel<RECIPE, FMT, true, AMAX, nh>;
    p.rc_cols = 64 * nh;
  }
  else if (!W2D && mask == PBS_COL) p.col = cast_col_kernel<RECIPE, FMT, RHT, SR, AMAX>;
  else if (mask == PBS_ROW) p.tile = cast_tile_kernel<RECIPE, FMT, true, false, W2D, false, SR, AMAX>;
  else if (mask == PBS_COL) p.tile = cast_tile_kernel<RECIPE, FMT, false, true, W2D, RHT, SR, AMAX>;
  else p.tile = cast_tile_kernel<RECIPE, FMT, true, true, W2D, false, SR, AMAX>;
  return p;
}

}  // namespace pbs

using namespace pbs;

// pbs_cast and pbs_rht_cast: `seed` keys stochastic rounding, `rht_seed`
// the Hadamard transform's signs.
static pbs_status cast_impl(pbs_recipe recipe, const void* x_bf16, int64_t rows, int64_t cols, pbs_format fmt,
                            int orient_mask, int weight_2d, int flags, uint64_t seed, uint64_t rht_seed,
                            const float* scale, float* amax_out, void* row_codes, void* row_scales,
                            void* col_codes, void* col_scales, hipStream_t stream) {
  PBS_REQUIRE(orient_mask >= 1 && orient_mask <= 3, PBS_ERR_INVALID_ARG,
              "pbs_cast: orient_mask must be PBS_ROW, PBS_COL or both");
  PBS_REQUIRE((flags & ~(PBS_FLAG_RHT16 | PBS_FLAG_SR)) == 0, PBS_ERR_INVALID_ARG,
              "pbs_cast: unknown flags %d", flags);
  PBS_REQUIRE(rows >= 0 && cols >= 0, PBS_ERR_SHAPE, "pbs_cast: negative shape");
  PBS_REQUIRE(rows % 16 == 0 && cols % 16 == 0, PBS_ERR_SHAPE,
              "pbs_cast: rows and cols must be multiples of 16 (got %lld x %lld)", (long long)rows,
              (long long)cols);
  const bool row = orient_mask & PBS_ROW, col = orient_mask & PBS_COL;
  const bool rht = flags & PBS_FLAG_RHT16, sr = flags & PBS_FLAG_SR;
  const bool w2d = weight_2d != 0;
  PBS_REQUIRE(rows * cols == 0 || x_bf16, PBS_ERR_INVALID_ARG, "pbs_cast: x is null");
  PBS_REQUIRE(((uintptr_t)x_bf16 & 15) == 0, PBS_ERR_INVALID_ARG, "pbs_cast: x not 16-byte aligned");
  PBS_REQUIRE(!row || row_codes, PBS_ERR_INVALID_ARG, "pbs_cast: row_codes is null");
  PBS_REQUIRE(!col || col_codes, PBS_ERR_INVALID_ARG, "pbs_cast: col_codes is null");
  PBS_REQUIRE(!row || ((uintptr_t)row_codes & 15) == 0, PBS_ERR_INVALID_ARG, "pbs_cast: row_codes not 16-byte aligned");
  PBS_REQUIRE(!col || ((uintptr_t)col_codes & 15) == 0, PBS_ERR_INVALID_ARG, "pbs_cast: col_codes not 16-byte aligned");
  PBS_REQUIRE(!rht && !sr || recipe == PBS_RECIPE_NVFP4 || recipe == PBS_RECIPE_MXFP4, PBS_ERR_UNSUPPORTED,
              "pbs_cast: RHT16 / SR flags apply to the NVFP4 and MXFP4 recipes only");
  PBS_REQUIRE(!rht || orient_mask == PBS_COL, PBS_ERR_UNSUPPORTED,
              "pbs_cast: RHT16 runs along the rows and produces the col copy only");
  PBS_REQUIRE(!w2d || recipe == PBS_RECIPE_FP8_BLOCK128 || recipe == PBS_RECIPE_FP8_BLOCK128_2D2D ||
                  recipe == PBS_RECIPE_FP8_BLOCK128_POW2 || recipe == PBS_RECIPE_NVFP4,
              PBS_ERR_UNSUPPORTED, "pbs_cast: 2D blocks exist for FP8_BLOCK128(_2D2D, _POW2) and NVFP4 only");
  PBS_REQUIRE(!(w2d && (rht || sr)), PBS_ERR_UNSUPPORTED,
              "pbs_cast: 2D weight blocks take neither RHT16 nor SR");
  PBS_REQUIRE(amax_out == nullptr || recipe == PBS_RECIPE_FP8_CURRENT || recipe == PBS_RECIPE_FP8_DELAYED,
              PBS_ERR_UNSUPPORTED, "pbs_cast: fused amax is for the per-tensor recipes");

  CastArgs a;
  a.x = (const bf16_t*)x_bf16;
  a.R = rows;
  a.C = cols;
  a.scale = scale;
  a.amax_out = (uint32_t*)amax_out;
  a.row_codes = (uint8_t*)row_codes;
  a.row_scales = row_scales;
  a.col_codes = (uint8_t*)col_codes;
  a.col_scales = col_scales;
  a.seed = seed;
  a.rht_seed = rht_seed;

  CastPick fn;
  const char* name = "";
  switch (recipe) {
    case PBS_RECIPE_FP8_CURRENT:
    case PBS_RECIPE_FP8_DELAYED: {
      PBS_REQUIRE(fmt == PBS_FMT_E4M3 || fmt == PBS_FMT_E5M2, PBS_ERR_UNSUPPORTED,
                  "pbs_cast: per-tensor FP8 takes E4M3 or E5M2");
      PBS_REQUIRE(scale, PBS_ERR_INVALID_ARG, "pbs_cast: per-tensor FP8 needs the device scale");
      const bool am = amax_out != nullptr;
      if (fmt == PBS_FMT_E4M3)
        fn = am ? pick_orient<R_TENSOR, F_E4M3, false, false, false, true>(orient_mask)
                : pick_orient<R_TENSOR, F_E4M3, false, false, false, false>(orient_mask);
      else
        fn = am ? pick_orient<R_TENSOR, F_E5M2, false, false, false, true>(orient_mask)
                : pick_orient<R_TENSOR, F_E5M2, false, false, false, false>(orient_mask);
      name = "cast_tensor_fp8";
      break;
    }
    case PBS_RECIPE_FP8_BLOCK128:
    case PBS_RECIPE_FP8_BLOCK128_1D1D:
    case PBS_RECIPE_FP8_BLOCK128_2D2D: {
      PBS_REQUIRE(fmt == PBS_FMT_E4M3, PBS_ERR_UNSUPPORTED, "pbs_cast: FP8_BLOCK128 takes E4M3");
      PBS_REQUIRE((!row || cols % 128 == 0) && (!col || rows % 128 == 0) &&
                      (!w2d || (rows % 128 == 0 && cols % 128 == 0)),
                  PBS_ERR_SHAPE, "pbs_cast: FP8_BLOCK128 needs the blocked dims to be multiples of 128");
      PBS_REQUIRE((!row || row_scales) && (!col || col_scales), PBS_ERR_INVALID_ARG,
                  "pbs_cast: block scales output is null");
      fn = w2d ? pick_orient<R_BLOCK128, F_E4M3, true, false, false, false>(orient_mask)
               : pick_orient<R_BLOCK128, F_E4M3, false, false, false, false>(orient_mask);
      name = "cast_block128";
      break;
    }
    case PBS_RECIPE_FP8_BLOCK128_POW2: {
      PBS_REQUIRE(fmt == PBS_FMT_E4M3, PBS_ERR_UNSUPPORTED, "pbs_cast: FP8_BLOCK128_POW2 takes E4M3");
      PBS_REQUIRE((!row || cols % 128 == 0) && (!col || rows % 128 == 0) &&
                      (!w2d || (rows % 128 == 0 && cols % 128 == 0)),
                  PBS_ERR_SHAPE, "pbs_cast: FP8_BLOCK128_POW2 needs the blocked dims to be multiples of 128");
      PBS_REQUIRE((!row || row_scales) && (!col || col_scales), PBS_ERR_INVALID_ARG,
                  "pbs_cast: block scales output is null");
      PBS_REQUIRE((!row || ((uintptr_t)row_scales & 3) == 0) && (!col || ((uintptr_t)col_scales & 3) == 0),
                  PBS_ERR_INVALID_ARG, "pbs_cast: FP8_BLOCK128_POW2 scale words must be 4-byte aligned");
      fn = w2d ? pick_orient<R_B128P2, F_E4M3, true, false, false, false>(orient_mask)
               : pick_orient<R_B128P2, F_E4M3, false, false, false, false>(orient_mask);
      name = "cast_block128_pow2";
      break;
    }
    case PBS_RECIPE_MXFP8: {
      PBS_REQUIRE(fmt == PBS_FMT_E4M3, PBS_ERR_UNSUPPORTED, "pbs_cast: MXFP8 takes E4M3");
      PBS_REQUIRE((!row || cols % 32 == 0) && (!col || rows % 32 == 0), PBS_ERR_SHAPE,
                  "pbs_cast: MXFP8 needs the blocked dim to be a multiple of 32");
      PBS_REQUIRE((!row || row_scales) && (!col || col_scales), PBS_ERR_INVALID_ARG,
                  "pbs_cast: block scales output is null");
      fn = pick_orient<R_MX, F_E4M3, false, false, false, false>(orient_mask);
      name = "cast_mxfp8";
      break;
    }
    case PBS_RECIPE_NVFP4: {
      PBS_REQUIRE(fmt == PBS_FMT_E2M1, PBS_ERR_UNSUPPORTED, "pbs_cast: NVFP4 takes E2M1");
      PBS_REQUIRE(scale, PBS_ERR_INVALID_ARG, "pbs_cast: NVFP4 needs the device S_enc");
      PBS_REQUIRE((!row || row_scales) && (!col || col_scales), PBS_ERR_INVALID_ARG,
                  "pbs_cast: block scales output is null");
      if (rht)
        fn = sr ? pick_orient<R_NV, F_E4M3, false, true, true, false>(orient_mask)
                : pick_orient<R_NV, F_E4M3, false, true, false, false>(orient_mask);
      else if (w2d)
        fn = pick_orient<R_NV, F_E4M3, true, false, false, false>(orient_mask);
      else
        fn = sr ? pick_orient<R_NV, F_E4M3, false, false, true, false>(orient_mask)
                : pick_orient<R_NV, F_E4M3, false, false, false, false>(orient_mask);
      name = "cast_nvfp4";
      break;
    }
    case PBS_RECIPE_MXFP4: {
      PBS_REQUIRE(fmt == PBS_FMT_E2M1, PBS_ERR_UNSUPPORTED, "pbs_cast: MXFP4 takes E2M1");
      PBS_REQUIRE((!row || cols % 32 == 0) && (!col || rows % 32 == 0), PBS_ERR_SHAPE,
                  "pbs_cast: MXFP4 needs the blocked dim to be a multiple of 32");
      PBS_REQUIRE((!row || row_scales) && (!col || col_scales), PBS_ERR_INVALID_ARG,
                  "pbs_cast: block scales output is null");
      if (rht)
        fn = sr ? pick_orient<R_MX4, F_E4M3, false, true, true, false>(orient_mask)
                : pick_orient<R_MX4, F_E4M3, false, true, false, false>(orient_mask);
      else
        fn = sr ? pick_orient<R_MX4, F_E4M3, false, false, true, false>(orient_mask)
                : pick_orient<R_MX4, F_E4M3, false, false, false, false>(orient_mask);
      name = "cast_mxfp4";
      break;
    }
    case PBS_RECIPE_FP8_CHANNEL: {
      PBS_REQUIRE(fmt == PBS_FMT_E4M3, PBS_ERR_UNSUPPORTED, "pbs_cast: FP8_CHANNEL takes E4M3");
      PBS_REQUIRE((!row || row_scales) && (!col || col_scales), PBS_ERR_INVALID_ARG,
                  "pbs_cast: channel scales output is null");
      PBS_REQUIRE((!row || ((uintptr_t)row_scales & 3) == 0) && (!col || ((uintptr_t)col_scales & 3) == 0),
                  PBS_ERR_INVALID_ARG, "pbs_cast: channel scales must be 4-byte aligned");
      return cast_channel(a, row, col, stream);
    }
    case PBS_RECIPE_BF16:
      return set_error(PBS_ERR_UNSUPPORTED, "pbs_cast: the BF16 recipe has no cast");
    default:
      return set_error(PBS_ERR_INVALID_ARG, "pbs_cast: unknown recipe %d", (int)recipe);
  }
  PBS_REQUIRE(!fn.tile || ceil_div(rows, TILE) <= 65535, PBS_ERR_SHAPE,
              "pbs_cast: 2D-block casts and two-copy casts with stochastic rounding take at most 65535 x 128 rows "
              "(got %lld)",
              (long long)rows);
  if (amax_out) hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, stream, (uint32_t*)amax_out);
  if (rows == 0 || cols == 0) return check_launch("pbs_cast");
  if (fn.row) {
    const int64_t nseg = rows * cols / 16;
    // one pass of the wave loop per wave (measured best); with fused amax
    // at most 1024 longer-lived workgroups: each ends in one same-address
    // atomic at most, and thousands of those queue behind each other
    const unsigned grid = (unsigned)std::min<int64_t>(ceil_div(nseg, 1024), amax_out ? 1024 : (1 << 20));
    log_dispatch("%s_row recipe=%d fmt=%d flags=%d rows=%lld cols=%lld grid=%u", name, (int)recipe, (int)fmt,
                 flags, (long long)rows, (long long)cols, grid);
    hipLaunchKernelGGL(fn.row, dim3(grid), dim3(256), 0, stream, a, nseg);
  } else if (fn.rc) {
    // a 1D grid of at most RC_GRID workgroups walking the 256 x 128 tiles
    // (each prefetches its next tile; with fused amax at most that many
    // same-address atomics end the pass)
    const int64_t ntiles = ceil_div(cols, fn.rc_cols) * ceil_div(rows, CT_R);
    const dim3 grid((unsigned)std::min<int64_t>(ntiles, RC_GRID), 1);
    log_dispatch("%s_%s recipe=%d fmt=%d rows=%lld cols=%lld grid=%u", name, row ? "rowcol" : "col", (int)recipe,
                 (int)fmt, (long long)rows, (long long)cols, grid.x);
    hipLaunchKernelGGL(fn.rc, grid, dim3(256), 0, stream, a);
  } else if (fn.col) {
    // a 1D grid over the tiles in row-major tile order, one tile per
    // workgroup; with fused amax at most 1024 workgroups walk the tiles (one
    // same-address atomic at most per workgroup)
    const int64_t ntiles = ceil_div(cols, CT_C) * ceil_div(rows, CT_R);
    const dim3 grid((unsigned)std::min<int64_t>(ntiles, amax_out ? 1024 : (int64_t)1 << 30), 1);
    log_dispatch("%s_col recipe=%d fmt=%d flags=%d rows=%lld cols=%lld grid=%u", name, (int)recipe,
                 (int)fmt, flags, (long long)rows, (long long)cols, grid.x);
    hipLaunchKernelGGL(fn.col, grid, dim3(256), 0, stream, a);
  } else {
    dim3 grid((unsigned)ceil_div(cols, TILE), (unsigned)ceil_div(rows, TILE));
    log_dispatch("%s recipe=%d fmt=%d orient=%d w2d=%d flags=%d rows=%lld cols=%lld grid=%ux%u", name,
                 (int)recipe, (int)fmt, orient_mask, (int)w2d, flags, (long long)rows, (long long)cols,
                 grid.x, grid.y);
    hipLaunchKernelGGL(fn.tile, grid, dim3(128), 0, stream, a);
  }
  return check_launch("pbs_cast");
}

// Sanity of every pointer argument is checked by cast_impl; the Wgrad
// operand of the 4-bit recipes is its transposed (col) copy.
extern "C" pbs_status pbs_cast(pbs_recipe recipe, const void* x_bf16, int64_t rows, int64_t cols,
                               pbs_format fmt, int orient_mask, int weight_2d, int flags,
                               uint64_t seed, const float* scale, float* amax_out, void* row_codes,
                               void* row_scales, void* col_codes, void* col_scales,
                               hipStream_t stream) {
  return cast_impl(recipe, x_bf16, rows, cols, fmt, orient_mask, weight_2d, flags, seed, seed, scale, amax_out,
                   row_codes, row_scales, col_codes, col_scales, stream);
}

extern "C" pbs_status pbs_rht_cast(pbs_recipe recipe, const void* x_bf16, int64_t rows, int64_t cols,
                                   uint64_t rht_seed, int stochastic, uint64_t sr_seed, const float* scale,
                                   void* col_codes, void* col_scales, hipStream_t stream) {
  PBS_REQUIRE(recipe == PBS_RECIPE_NVFP4 || recipe == PBS_RECIPE_MXFP4, PBS_ERR_UNSUPPORTED,
              "pbs_rht_cast: the Hadamard transform applies to the NVFP4 and MXFP4 recipes only");
  PBS_REQUIRE(stochastic == 0 || stochastic == 1, PBS_ERR_INVALID_ARG, "pbs_rht_cast: stochastic must be 0 or 1");
  PBS_REQUIRE(rows % 16 == 0, PBS_ERR_SHAPE, "pbs_rht_cast: rows must be a multiple of 16 (got %lld)",
              (long long)rows);
  const int flags = PBS_FLAG_RHT16 | (stochastic ? PBS_FLAG_SR : 0);
  return cast_impl(recipe, x_bf16, rows, cols, PBS_FMT_E2M1, PBS_COL, 0, flags, sr_seed, rht_seed, scale, nullptr,
                   nullptr, nullptr, col_codes, col_scales, stream);
}

// ---------------------------------------------------------------------------
// Test hook: the device's stochastic E2M1 rounding on given values and
// random words, one 4-bit code (sign in bit 3) per output byte.
// ---------------------------------------------------------------------------
namespace pbs {
__global__ void sr_debug_kernel(const float* v, const uint32_t* r, uint8_t* out, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = (uint8_t)sr_e2m1(v[i], r[i]);
}
}  // namespace pbs

extern "C" pbs_status pbs_debug_sr_encode(const float* v, const uint32_t* r, uint8_t* codes, int64_t n,
                                          hipStream_t stream) {
  PBS_REQUIRE(n >= 0, PBS_ERR_SHAPE, "pbs_debug_sr_encode: negative length");
  PBS_REQUIRE(n == 0 || (v && r && codes), PBS_ERR_INVALID_ARG, "pbs_debug_sr_encode: null pointer");
  PBS_REQUIRE(((uintptr_t)v & 3) == 0 && ((uintptr_t)r & 3) == 0, PBS_ERR_INVALID_ARG,
              "pbs_debug_sr_encode: v and r must be 4-byte aligned");
  if (n == 0) return PBS_OK;
  const unsigned grid = (unsigned)std::min<int64_t>(ceil_div(n, 256), 4096);
  log_dispatch("sr_debug n=%lld grid=%u", (long long)n, grid);
  hipLaunchKernelGGL(sr_debug_kernel, dim3(grid), dim3(256), 0, stream, v, r, codes, n);
  return check_launch("pbs_debug_sr_encode");
}
