// GEMM kernels for every recipe on the gfx950 matrix cores.
//
// C[M, N] = sum_k A[m, k] * B[n, k], fp32 accumulation, for the Fprop /
// Dgrad / Wgrad products of a linear layer ("How to optimize
// Transformer-based models for low-precision training", "Model
// configuration and training inputs" and "Using autocast mode vs
// pre-quantized mode").
//
// Mapping of each recipe onto the gfx950 MFMA instructions:
//  BF16        v_mfma_f32_32x32x16_bf16.  Operands may be stored
//              contraction-contiguous or, for the Dgrad / Wgrad products of
//              natural-layout tensors, MN-contiguous; MN-contiguous tiles are
//              transposed in registers (4x8 bf16 blocks) on their way into
//              LDS, so the MFMA always reads contraction-contiguous rows.
//  FP8 per-tensor  v_mfma_f32_32x32x64_f8f6f4 (format per operand: E4M3 or
//              E5M2), scales applied once in the epilogue.
//  FP8 1x128 / 128x128  the same instruction; each 128-long slice of the
//              contraction accumulates into fresh registers, then is added
//              into the result times a_scale[m] * b_scale[n] (fp32 block
//              scales are not powers of two, so they cannot ride on the
//              instruction's E8M0 scale).
//  MXFP8       v_mfma_scale_f32_32x32x64_f8f6f4: each K=64 step covers two
//              MX blocks; the two lanes that hold a row (or column) each
//              supply the E8M0 scale of one of its blocks, and the hardware
//              applies it to that block's 32 products.
//  NVFP4       E2M1 x E4M3 block scale has up to 6 significant bits, more
//              than any 4-, 6- or 8-bit MFMA input holds, so the operands are
//              decoded exactly into fp16 (E2M1 -> fp16 by conversion, times
//              the block scale by an exact fp16 multiply: the product needs
//              <= 6 bits and lies in [2^-10, 2688]) on their way into LDS,
//              and the product runs on v_mfma_f32_32x32x16_f16.  The two
//              fp32 tensor scales are applied in the epilogue.
//
// Tiling: 128 x 128 output tile per workgroup of 256 threads (4 waves in a
// 2 x 2 grid, 64 x 64 per wave, 2 x 2 MFMA 32x32 tiles per wave).  Each
// K stage moves 128 bytes per operand row (64 bf16 / fp16, 128 fp8) through
// a double-buffered LDS tile whose 16-byte chunks are XOR-swizzled by row
// so that the MFMA fragment reads (ds_read_b128) are conflict-free.
#include "device.hpp"
#include "host.hpp"

namespace pbs {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

enum { OP_BF16 = 0, OP_F16 = 1, OP_FP8 = 2 };                 // what the MFMA consumes
enum { LD_KMAJOR = 0, LD_MNMAJOR = 1, LD_NVFP4 = 2 };         // how a tile reaches LDS
enum { SC_NONE = 0, SC_TENSOR = 1, SC_MX = 2, SC_BLK = 3, SC_NV = 4 };

constexpr int BM = 128, BN = 128, NTHR = 256;
constexpr int ROWB = 128;               // bytes per LDS row per K stage
constexpr int TILEB = BM * ROWB;        // 16 KB per operand per stage

struct GemmArgs {
  const uint8_t* A;
  const uint8_t* B;
  const uint8_t* a_scale;
  const uint8_t* b_scale;
  const float* a_ts;
  const float* b_ts;
  void* C;
  int M, N, K;            // GEMM dims, K in elements
  int64_t lda, ldb;       // bytes between stored rows of A / B
  int ldc;                // elements between rows of C
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * ROWB + ((chunk ^ (row & 7)) << 4); }

// ---------------------------------------------------------------------------
// Global -> register -> LDS staging, one operand.
//   rows0: first tile row (M or N index), nrows: valid rows (M or N)
// ---------------------------------------------------------------------------
template <int LD, bool SCALE2D>
struct Stage {
  uint4 v[4];
  uint32_t s;             // NVFP4 block scale bytes (2)
};

// K-major: tile row r, 16-byte chunk c: thread t loads chunks t + 256 i.
template <int LD, bool SCALE2D>
__device__ __forceinline__ void load_stage(Stage<LD, SCALE2D>& st, const uint8_t* base, int64_t ld,
                                           int rows0, int nrows, int kt, int K,
                                           const uint8_t* scale) {
  const int t = threadIdx.x;
  if (LD == LD_KMAJOR) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = t + NTHR * i;
      int row = rows0 + (q >> 3);
      row = row < nrows ? row : nrows - 1;
      st.v[i] = *(const uint4*)(base + (int64_t)row * ld + (int64_t)kt * ROWB + ((q & 7) << 4));
    }
  } else if (LD == LD_MNMAJOR) {
    // stored [K][MN], ld = bytes per k row; this thread: k rows 4*kq..+3, mn 8*mq..+7
    const int kq = t >> 4, mq = t & 15;
    int mn = rows0 + 8 * mq;
    mn = mn < nrows ? mn : nrows - 8;
    const int64_t k = (int64_t)kt * 64 + 4 * kq;
#pragma unroll
    for (int i = 0; i < 4; ++i) st.v[i] = *(const uint4*)(base + (k + i) * ld + (int64_t)mn * 2);
  } else {  // LD_NVFP4: row t/2, 32 values (16 bytes) at K offset 64 kt + 32 (t & 1)
    const int r = t >> 1, half = t & 1;
    int row = rows0 + r;
    row = row < nrows ? row : nrows - 1;
    st.v[0] = *(const uint4*)(base + (int64_t)row * ld + (int64_t)kt * 32 + half * 16);
    const int64_t kb = ((int64_t)kt * 64 + 32 * half) / 16;          // first of two blocks
    const int64_t srow = SCALE2D ? row / 16 : row;
    st.s = *(const uint16_t*)(scale + srow * (K / 16) + kb);
  }
}

template <int LD, bool SCALE2D>
__device__ __forceinline__ void store_stage(const Stage<LD, SCALE2D>& st, uint8_t* lds) {
  const int t = threadIdx.x;
  if (LD == LD_KMAJOR) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = t + NTHR * i;
      *(uint4*)(lds + swz(q >> 3, q & 7)) = st.v[i];
    }
  } else if (LD == LD_MNMAJOR) {
    const int kq = t >> 4, mq = t & 15;
    const uint32_t w0[4] = {st.v[0].x, st.v[0].y, st.v[0].z, st.v[0].w};
    const uint32_t w1[4] = {st.v[1].x, st.v[1].y, st.v[1].z, st.v[1].w};
    const uint32_t w2[4] = {st.v[2].x, st.v[2].y, st.v[2].z, st.v[2].w};
    const uint32_t w3[4] = {st.v[3].x, st.v[3].y, st.v[3].z, st.v[3].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // mn row 8 mq + i gets (k 4kq .. 4kq+3) = element i of each loaded row
      const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
      uint2 o;
      o.x = __builtin_amdgcn_perm(w1[i >> 1], w0[i >> 1], sel);
      o.y = __builtin_amdgcn_perm(w3[i >> 1], w2[i >> 1], sel);
      const int row = 8 * mq + i;
      *(uint2*)(lds + swz(row, kq >> 1) + ((kq & 1) << 3)) = o;
    }
  } else {  // LD_NVFP4: decode 32 E2M1 values to fp16 times their block scale
    const int r = t >> 1, half = t & 1;
    const uint32_t w[4] = {st.v[0].x, st.v[0].y, st.v[0].z, st.v[0].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t dcode = (st.s >> (8 * (j >> 1))) & 0x7Fu;   // words 0,1: block 0; 2,3: block 1
      const _Float16 dh = (_Float16)dec_e4m3_pos(dcode);           // exact: E4M3 fits fp16
      const f16x2 dd = {dh, dh};
      f16x2 h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[j], 1.0f, 0) * dd;
      f16x2 h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[j], 1.0f, 1) * dd;
      f16x2 h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[j], 1.0f, 2) * dd;
      f16x2 h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[j], 1.0f, 3) * dd;
      uint4 o;
      o.x = __builtin_bit_cast(uint32_t, h0);
      o.y = __builtin_bit_cast(uint32_t, h1);
      o.z = __builtin_bit_cast(uint32_t, h2);
      o.w = __builtin_bit_cast(uint32_t, h3);
      *(uint4*)(lds + swz(r, half * 4 + j)) = o;
    }
  }
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
template <int OP, int LDA, int LDB, int SC, int AFMT, int BFMT, bool B2D, bool OUT_BF16>
__global__ __launch_bounds__(NTHR) void gemm_kernel(GemmArgs g) {
  __shared__ __align__(16) uint8_t lds[2][2][TILEB];     // [stage][A/B]
  __shared__ __align__(16) uint32_t lds_sc[2][2][BM];    // [stage][A/B][row] MX dwords / block fp32

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int KST = (OP == OP_FP8) ? 128 : 64;              // K elements per stage
  const int nk = g.K / KST;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  Stage<LDA, false> sa;
  Stage<LDB, B2D> sb;
  uint32_t sca = 0, scb = 0;

  auto load_scales = [&](int kt) {
    if (SC == SC_MX) {
      const int r = t & 127;
      if (t < 128) {
        int row = m0 + r; row = row < g.M ? row : g.M - 1;
        sca = *(const uint32_t*)(g.a_scale + (int64_t)row * (g.K / 32) + kt * 4);
      } else {
        int row = n0 + r; row = row < g.N ? row : g.N - 1;
        scb = *(const uint32_t*)(g.b_scale + (int64_t)row * (g.K / 32) + kt * 4);
      }
    } else if (SC == SC_BLK) {
      const int r = t & 127;
      const float* as = (const float*)g.a_scale;
      const float* bs = (const float*)g.b_scale;
      if (t < 128) {
        int row = m0 + r; row = row < g.M ? row : g.M - 1;
        sca = __float_as_uint(as[(int64_t)row * (g.K / 128) + kt]);
      } else {
        int row = n0 + r; row = row < g.N ? row : g.N - 1;
        scb = __float_as_uint(B2D ? bs[(int64_t)(row / 128) * (g.K / 128) + kt]
                                  : bs[(int64_t)row * (g.K / 128) + kt]);
      }
    }
  };
  auto store_scales = [&](int buf) {
    if (SC == SC_MX || SC == SC_BLK) {
      if (t < 128) lds_sc[buf][0][t] = sca;
      else lds_sc[buf][1][t - 128] = scb;
    }
  };

  load_stage<LDA, false>(sa, g.A, g.lda, m0, g.M, 0, g.K, g.a_scale);
  load_stage<LDB, B2D>(sb, g.B, g.ldb, n0, g.N, 0, g.K, g.b_scale);
  load_scales(0);
  store_stage<LDA, false>(sa, lds[0][0]);
  store_stage<LDB, B2D>(sb, lds[0][1]);
  store_scales(0);
  __syncthreads();

  const int lr = lane & 31, lg = lane >> 5;     // row within a 32-tile, K group
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) {
      load_stage<LDA, false>(sa, g.A, g.lda, m0, g.M, kt + 1, g.K, g.a_scale);
      load_stage<LDB, B2D>(sb, g.B, g.ldb, n0, g.N, kt + 1, g.K, g.b_scale);
      load_scales(kt + 1);
    }
    const uint8_t* la = lds[buf][0];
    const uint8_t* lb = lds[buf][1];

    if (OP == OP_BF16 || OP == OP_F16) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint4 fa[2], fb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) fa[i] = *(const uint4*)(la + swz(wm * 64 + 32 * i + lr, 2 * s + lg));
#pragma unroll
        for (int j = 0; j < 2; ++j) fb[j] = *(const uint4*)(lb + swz(wn * 64 + 32 * j + lr, 2 * s + lg));
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            if (OP == OP_BF16)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(bf16x8, fa[i]), __builtin_bit_cast(bf16x8, fb[j]), acc[i][j], 0, 0, 0);
            else
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                  __builtin_bit_cast(f16x8, fa[i]), __builtin_bit_cast(f16x8, fb[j]), acc[i][j], 0, 0, 0);
          }
      }
    } else {
      // OP_FP8: two K=64 steps per stage.  Operand layout of the 32x32x64
      // f8f6f4 instruction (8-bit formats): lane l holds row (or column)
      // l % 32; its bytes 0-15 are K 16 g .. 16 g + 15 and bytes 16-31 are
      // K 32 + 16 g .. 32 + 16 g + 15, g = l / 32.  The E8M0 scale that lane
      // l supplies applies to K block g (K 32 g .. 32 g + 31) of its row.
      // So lane group g reads 16-byte chunks g and 2 + g of each 64-byte step,
      // and supplies the scale of MX block 2 s + g of the stage.
      f32x16 part[2][2];
      if (SC == SC_BLK) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) part[i][j][r] = 0.0f;
      }
      uint32_t mxa[2] = {0, 0}, mxb[2] = {0, 0};
      if (SC == SC_MX) {
#pragma unroll
        for (int i = 0; i < 2; ++i) mxa[i] = lds_sc[buf][0][wm * 64 + 32 * i + lr];
#pragma unroll
        for (int j = 0; j < 2; ++j) mxb[j] = lds_sc[buf][1][wn * 64 + 32 * j + lr];
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        i32x8 fa[2], fb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int row = wm * 64 + 32 * i + lr;
          const uint4 lo = *(const uint4*)(la + swz(row, 4 * s + lg));
          const uint4 hi = *(const uint4*)(la + swz(row, 4 * s + 2 + lg));
          fa[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int row = wn * 64 + 32 * j + lr;
          const uint4 lo = *(const uint4*)(lb + swz(row, 4 * s + lg));
          const uint4 hi = *(const uint4*)(lb + swz(row, 4 * s + 2 + lg));
          fb[j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            if (SC == SC_MX) {
              // this lane's block within the stage: 2 s + lg (byte of the row's dword)
              const int sa_ = (int)((mxa[i] >> (8 * (2 * s + lg))) & 0xFFu);
              const int sb_ = (int)((mxb[j] >> (8 * (2 * s + lg))) & 0xFFu);
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], AFMT,
                                                                           BFMT, 0, sa_, 0, sb_);
            } else if (SC == SC_BLK) {
              part[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], part[i][j], AFMT,
                                                                            BFMT, 0, 0, 0, 0);
            } else {
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], AFMT,
                                                                           BFMT, 0, 0, 0, 0);
            }
          }
      }
      if (SC == SC_BLK) {
        // acc += part * (a_scale[row] * b_scale[col]) for this 128-long K block
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float sbv = __uint_as_float(lds_sc[buf][1][wn * 64 + 32 * j + lr]);
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = wm * 64 + 32 * i + (r >> 2) * 8 + lg * 4 + (r & 3);
              const float f = __uint_as_float(lds_sc[buf][0][row]) * sbv;
              acc[i][j][r] = __builtin_fmaf(part[i][j][r], f, acc[i][j][r]);
            }
        }
      }
    }

    if (kt + 1 < nk) {
      store_stage<LDA, false>(sa, lds[buf ^ 1][0]);
      store_stage<LDB, B2D>(sb, lds[buf ^ 1][1]);
      store_scales(buf ^ 1);
    }
    __syncthreads();
  }

  // Epilogue.
  float post = 1.0f;
  if (SC == SC_TENSOR || SC == SC_NV) post = (*g.a_ts) * (*g.b_ts);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + 32 * j + lr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 64 + 32 * i + (r >> 2) * 8 + lg * 4 + (r & 3);
        if (row < g.M && col < g.N) {
          float v = acc[i][j][r];
          if (SC == SC_TENSOR || SC == SC_NV) v *= post;
          if (OUT_BF16)
            ((uint16_t*)g.C)[(int64_t)row * g.ldc + col] = (uint16_t)f32_to_bf16_rne(v);
          else
            ((float*)g.C)[(int64_t)row * g.ldc + col] = v;
        }
      }
    }
}

__global__ void zero_c_kernel(uint8_t* c, int64_t bytes) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < bytes; i += (int64_t)gridDim.x * blockDim.x)
    c[i] = 0;
}

typedef void (*gemm_fn)(GemmArgs);

template <int OP, int LDA, int LDB, int SC, int AFMT, int BFMT, bool B2D>
static gemm_fn pick_out(bool bf16_out) {
  return bf16_out ? gemm_kernel<OP, LDA, LDB, SC, AFMT, BFMT, B2D, true>
                  : gemm_kernel<OP, LDA, LDB, SC, AFMT, BFMT, B2D, false>;
}

template <int SC, bool B2D>
static gemm_fn pick_fp8(int afmt, int bfmt, bool bf16_out) {
  if (afmt == 0 && bfmt == 0) return pick_out<OP_FP8, LD_KMAJOR, LD_KMAJOR, SC, 0, 0, B2D>(bf16_out);
  if (afmt == 1 && bfmt == 0) return pick_out<OP_FP8, LD_KMAJOR, LD_KMAJOR, SC, 1, 0, B2D>(bf16_out);
  if (afmt == 0 && bfmt == 1) return pick_out<OP_FP8, LD_KMAJOR, LD_KMAJOR, SC, 0, 1, B2D>(bf16_out);
  return pick_out<OP_FP8, LD_KMAJOR, LD_KMAJOR, SC, 1, 1, B2D>(bf16_out);
}

}  // namespace pbs

using namespace pbs;

extern "C" pbs_status pbs_gemm(pbs_recipe recipe, pbs_layout layout, int64_t M, int64_t N, int64_t K,
                               const void* A, pbs_format a_fmt, const void* a_scale,
                               const float* a_tensor_scale, const void* B, pbs_format b_fmt,
                               const void* b_scale, const float* b_tensor_scale, void* C,
                               pbs_format c_fmt, hipStream_t stream) {
  PBS_REQUIRE(layout >= PBS_FPROP && layout <= PBS_WGRAD, PBS_ERR_INVALID_ARG, "pbs_gemm: unknown layout %d",
              (int)layout);
  PBS_REQUIRE(c_fmt == PBS_FMT_F32 || c_fmt == PBS_FMT_BF16, PBS_ERR_UNSUPPORTED,
              "pbs_gemm: output format must be F32 or BF16");
  PBS_REQUIRE(M >= 0 && N >= 0 && K >= 0, PBS_ERR_SHAPE, "pbs_gemm: negative shape");
  PBS_REQUIRE(M % 16 == 0 && N % 16 == 0, PBS_ERR_SHAPE,
              "pbs_gemm: M and N must be multiples of 16 (got %lld, %lld)", (long long)M, (long long)N);
  PBS_REQUIRE(M <= (1 << 30) && N <= (1 << 30) && K <= (1 << 30), PBS_ERR_SHAPE, "pbs_gemm: dims too large");
  PBS_REQUIRE(M * N == 0 || C, PBS_ERR_INVALID_ARG, "pbs_gemm: C is null");
  const bool bf16_out = c_fmt == PBS_FMT_BF16;
  if (M == 0 || N == 0) return PBS_OK;
  if (K == 0) {
    const int64_t bytes = M * N * (bf16_out ? 2 : 4);
    hipLaunchKernelGGL(zero_c_kernel, dim3(1024), dim3(256), 0, stream, (uint8_t*)C, bytes);
    return check_launch("pbs_gemm");
  }
  PBS_REQUIRE(A && B, PBS_ERR_INVALID_ARG, "pbs_gemm: A or B is null");
  PBS_REQUIRE(((uintptr_t)A & 15) == 0 && ((uintptr_t)B & 15) == 0, PBS_ERR_INVALID_ARG,
              "pbs_gemm: A and B must be 16-byte aligned");

  GemmArgs g;
  g.A = (const uint8_t*)A;
  g.B = (const uint8_t*)B;
  g.a_scale = (const uint8_t*)a_scale;
  g.b_scale = (const uint8_t*)b_scale;
  g.a_ts = a_tensor_scale;
  g.b_ts = b_tensor_scale;
  g.C = C;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.ldc = (int)N;

  gemm_fn fn = nullptr;
  const char* name = "";
  const bool w2d = layout != PBS_WGRAD;     // weights carry 2D block scales
  switch (recipe) {
    case PBS_RECIPE_BF16: {
      PBS_REQUIRE(a_fmt == PBS_FMT_BF16 && b_fmt == PBS_FMT_BF16, PBS_ERR_UNSUPPORTED,
                  "pbs_gemm: BF16 recipe takes BF16 operands");
      PBS_REQUIRE(K % 64 == 0, PBS_ERR_SHAPE, "pbs_gemm: BF16 needs K %% 64 == 0");
      if (layout == PBS_FPROP) {
        g.lda = K * 2; g.ldb = K * 2;
        fn = pick_out<OP_BF16, LD_KMAJOR, LD_KMAJOR, SC_NONE, 0, 0, false>(bf16_out);
      } else if (layout == PBS_DGRAD) {
        g.lda = K * 2; g.ldb = N * 2;               // B = W stored [K, N]
        fn = pick_out<OP_BF16, LD_KMAJOR, LD_MNMAJOR, SC_NONE, 0, 0, false>(bf16_out);
      } else {
        g.lda = M * 2; g.ldb = N * 2;               // A = X stored [K, M], B = dY stored [K, N]
        fn = pick_out<OP_BF16, LD_MNMAJOR, LD_MNMAJOR, SC_NONE, 0, 0, false>(bf16_out);
      }
      name = "gemm_bf16";
      break;
    }
    case PBS_RECIPE_FP8_CURRENT:
    case PBS_RECIPE_FP8_DELAYED: {
      PBS_REQUIRE((a_fmt == PBS_FMT_E4M3 || a_fmt == PBS_FMT_E5M2) &&
                      (b_fmt == PBS_FMT_E4M3 || b_fmt == PBS_FMT_E5M2),
                  PBS_ERR_UNSUPPORTED, "pbs_gemm: per-tensor FP8 takes E4M3 / E5M2 operands");
      PBS_REQUIRE(a_tensor_scale && b_tensor_scale, PBS_ERR_INVALID_ARG,
                  "pbs_gemm: per-tensor FP8 needs both tensor scales");
      PBS_REQUIRE(K % 128 == 0, PBS_ERR_SHAPE, "pbs_gemm: FP8 needs K %% 128 == 0");
      g.lda = K; g.ldb = K;
      fn = pick_fp8<SC_TENSOR, false>(a_fmt == PBS_FMT_E5M2, b_fmt == PBS_FMT_E5M2, bf16_out);
      name = "gemm_fp8_tensor";
      break;
    }
    case PBS_RECIPE_FP8_BLOCK128: {
      PBS_REQUIRE(a_fmt == PBS_FMT_E4M3 && b_fmt == PBS_FMT_E4M3, PBS_ERR_UNSUPPORTED,
                  "pbs_gemm: FP8_BLOCK128 takes E4M3 operands");
      PBS_REQUIRE(a_scale && b_scale, PBS_ERR_INVALID_ARG, "pbs_gemm: block scales are null");
      PBS_REQUIRE(K % 128 == 0, PBS_ERR_SHAPE, "pbs_gemm: FP8_BLOCK128 needs K %% 128 == 0");
      PBS_REQUIRE(!w2d || N % 128 == 0, PBS_ERR_SHAPE, "pbs_gemm: 128x128 weight blocks need N %% 128 == 0");
      g.lda = K; g.ldb = K;
      fn = w2d ? pick_out<OP_FP8, LD_KMAJOR, LD_KMAJOR, SC_BLK, 0, 0, true>(bf16_out)
               : pick_out<OP_FP8, LD_KMAJOR, LD_KMAJOR, SC_BLK, 0, 0, false>(bf16_out);
      name = "gemm_fp8_block128";
      break;
    }
    case PBS_RECIPE_MXFP8: {
      PBS_REQUIRE(a_fmt == PBS_FMT_E4M3 && b_fmt == PBS_FMT_E4M3, PBS_ERR_UNSUPPORTED,
                  "pbs_gemm: MXFP8 takes E4M3 operands");
      PBS_REQUIRE(a_scale && b_scale, PBS_ERR_INVALID_ARG, "pbs_gemm: block scales are null");
      PBS_REQUIRE(K % 128 == 0, PBS_ERR_SHAPE, "pbs_gemm: MXFP8 needs K %% 128 == 0");
      g.lda = K; g.ldb = K;
      fn = pick_out<OP_FP8, LD_KMAJOR, LD_KMAJOR, SC_MX, 0, 0, false>(bf16_out);
      name = "gemm_mxfp8";
      break;
    }
    case PBS_RECIPE_NVFP4: {
      PBS_REQUIRE(a_fmt == PBS_FMT_E2M1 && b_fmt == PBS_FMT_E2M1, PBS_ERR_UNSUPPORTED,
                  "pbs_gemm: NVFP4 takes E2M1 operands");
      PBS_REQUIRE(a_scale && b_scale && a_tensor_scale && b_tensor_scale, PBS_ERR_INVALID_ARG,
                  "pbs_gemm: NVFP4 needs block and tensor scales");
      PBS_REQUIRE(K % 64 == 0, PBS_ERR_SHAPE, "pbs_gemm: NVFP4 needs K %% 64 == 0");
      PBS_REQUIRE(((uintptr_t)a_scale & 1) == 0 && ((uintptr_t)b_scale & 1) == 0, PBS_ERR_INVALID_ARG,
                  "pbs_gemm: NVFP4 block scales must be 2-byte aligned");
      g.lda = K / 2; g.ldb = K / 2;
      fn = w2d ? pick_out<OP_F16, LD_NVFP4, LD_NVFP4, SC_NV, 0, 0, true>(bf16_out)
               : pick_out<OP_F16, LD_NVFP4, LD_NVFP4, SC_NV, 0, 0, false>(bf16_out);
      name = "gemm_nvfp4";
      break;
    }
    default:
      return set_error(PBS_ERR_INVALID_ARG, "pbs_gemm: unknown recipe %d", (int)recipe);
  }
  dim3 grid((unsigned)ceil_div(N, BN), (unsigned)ceil_div(M, BM));
  log_dispatch("%s layout=%d M=%lld N=%lld K=%lld out=%s grid=%ux%u", name, (int)layout, (long long)M,
               (long long)N, (long long)K, bf16_out ? "bf16" : "f32", grid.x, grid.y);
  hipLaunchKernelGGL(fn, grid, dim3(NTHR), 0, stream, g);
  return check_launch("pbs_gemm");
}
