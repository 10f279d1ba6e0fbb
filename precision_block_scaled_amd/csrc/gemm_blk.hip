// Sub-channel FP8 GEMM: 1x128 or 128x128 fp32 block scales on either operand
// ("Faster training throughput in FP8 precision with NVIDIA NeMo",
// "Scaling recipe granularity": 1x128 activations and gradients with 128x128
// weights, and the other block pairings).  A 128x128-block operand stores one
// scale per 128 rows; the kernel reads it through the same per-row path.
//
//   C[m, n] = sum_kb (sum_{k in kb} A[m, k] B[n, k]) * a_scale[m, kb] * b_scale[n, kb]
//
// The fp32 block scales are not powers of two, so they cannot ride on the
// matrix instruction's E8M0 scale: every 128-long K block is multiplied on
// the matrix cores into fresh registers (two v_mfma_f32_32x32x64_f8f6f4 per
// 32x32 tile) and folded into the result by the vector unit, one fp32 FMA
// per output value and block.  That fold, not the matrix core, bounds the
// recipe unless it costs no more than the products it folds.
//
// So this kernel keeps everything the fold touches in VGPRs: a 256 x 128
// output tile per workgroup, 4 waves of 128 x 64 (2 x 2), 128 accumulators
// per lane, and the MFMAs write their partial products to VGPRs (this file
// is built with -amdgpu-mfma-vgpr-form).  Per wave and K block: 16 MFMAs
// (1024 matrix-core cycles) against 128 FMAs, plus 64 scale products for
// 128x128 weight blocks (the wave's 64 columns share one weight scale) or
// 128 for 1x128 Wgrad blocks.  The fold of tile t-1 runs while tile t
// multiplies.
//
// Staging: three LDS stage buffers of 48 KB (A 256 rows, B 128 rows, 128 B
// each, swizzled as in the other GEMMs) and a 3-deep scale-row ring, loads
// for stage k+2 spread over the MFMAs of stage k, one barrier per stage.
#include "device.hpp"
#include "gemm_common.hpp"
#include "host.hpp"

#include <type_traits>

namespace pbs {

constexpr int KB_BN = 128;                         // output columns per workgroup
constexpr int KB_TB = KB_BN * ROWB;                // 16 KB of B per stage
constexpr int KB_STAGE = TILEB + KB_TB;            // 48 KB per stage
constexpr int KB_NSTAGE = 3;
constexpr int KB_RING = KB_NSTAGE * KB_STAGE;      // scale ring after the stage buffers
constexpr int KB_NSLOT = 3;
constexpr int KB_SLOT = (BM + KB_BN + KB_BN) * 4;  // a_scale[256], b_scale[128], a sink for waves 2-3
constexpr int KB_STG_BF16 = 272;                   // epilogue staging pitch, bf16 (256 rows)
constexpr int KB_STG_F32 = 528;                    // epilogue staging pitch, fp32 (128 rows a pass)
constexpr int KB_SMEM = cmax(KB_RING + KB_NSLOT * KB_SLOT, cmax(256 * KB_STG_BF16, 128 * KB_STG_F32));
constexpr int KB_VM_TILES = 8 + 4;                 // tile loads per lane per stage: A, B

// B tile: 128 rows, 4 loads per lane; load i of wave w fills rows
// 32 w + 8 i .. + 7 (same chunk ownership as Direct).
struct Direct4 {
  const uint8_t* base;
  uint32_t off[4];
};

__device__ __forceinline__ void direct4_init(Direct4& d, const uint8_t* p, int64_t ld, int rows0, int nrows, int w) {
  const int lane = threadIdx.x & 63;
  d.base = p + (int64_t)rows0 * ld;
  const int lim = nrows - rows0 - 1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int trow = 32 * w + 8 * i + (lane >> 3);
    const int lc = (lane & 7) ^ swz_key(trow);
    const int r = trow < lim ? trow : lim;
    d.off[i] = (uint32_t)r * (uint32_t)ld + (uint32_t)(lc << 4);
  }
}

__device__ __forceinline__ void direct4_item(const Direct4& d, int kt, uint8_t* tile, int w, int i) {
  const uint8_t* g = d.base + (int64_t)kt * ROWB;
  __builtin_amdgcn_global_load_lds(g + d.off[i], (lds_ptr_t)(tile + (w * 4 + i) * 1024), 16, 0, 0);
}

// Epilogue.  The MFMAs compute each 32 x 32 tile transposed (B rows as the
// instruction's rows): lane (lr, lg) of tile (i, j) holds row
// m = 128 wm + 32 i + lr and columns n = 64 wn + 32 j + 8 q + 4 lg + {0..3}
// in values 4 q .. 4 q + 3.  Those go through LDS (4 consecutive columns per
// store) and every lane then writes 16 contiguous bytes of C.
template <bool OUT_BF16>
__device__ __forceinline__ void store_blk(f32x16 (&acc)[4][2], const GemmArgs& g, uint8_t* smem, int m0, int n0,
                                          int w, int wm, int wn, int lane) {
  const int lr = lane & 31, lg = lane >> 5;
  const bool full = (m0 + BM <= g.M) && (n0 + KB_BN <= g.N);
  if constexpr (OUT_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = wm * 128 + 32 * i + lr;
          const int colb = (wn * 64 + 32 * j + 8 * q + 4 * lg) * 2;
          *(uint2*)(smem + row * KB_STG_BF16 + colb) =
              make_uint2(pk_bf16(acc[i][j][4 * q], acc[i][j][4 * q + 1]), pk_bf16(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]));
        }
    __syncthreads();
    const int ch = lane & 15;
    uint32_t mx = 0;
#pragma unroll 4
    for (int it = 0; it < 16; ++it) {
      const int s = 64 * w + 4 * it + (lane >> 4);
      const uint4 val = *(const uint4*)(smem + s * KB_STG_BF16 + ch * 16);
      const int grow = m0 + s, gcol = n0 + ch * 8;
      if (full || (grow < g.M && gcol < g.N)) {
        *(uint4*)((uint16_t*)g.C + (int64_t)grow * g.ldc + gcol) = val;
        if (g.c_amax) {
          const uint32_t a = absmax_bf16x8(val);
          mx = mx > a ? mx : a;
        }
      }
    }
    if (g.c_amax) amax_fold_wg(mx, g.c_amax, smem);
  } else {
    uint32_t mx = 0;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      if (wm == p) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int row = 32 * i + lr;
              const int col = wn * 64 + 32 * j + 8 * q + 4 * lg;
              *(float4*)(smem + row * KB_STG_F32 + col * 4) =
                  make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
            }
      }
      __syncthreads();
#pragma unroll 4
      for (int it = 0; it < 16; ++it) {
        const int s = 32 * w + 2 * it + (lane >> 5);
        const uint4 val = *(const uint4*)(smem + s * KB_STG_F32 + (lane & 31) * 16);
        const int grow = m0 + 128 * p + s, gcol = n0 + (lane & 31) * 4;
        if (full || (grow < g.M && gcol < g.N)) {
          *(uint4*)((float*)g.C + (int64_t)grow * g.ldc + gcol) = val;
          if (g.c_amax) {
            const uint32_t a = absmax_f32x4(val);
            mx = mx > a ? mx : a;
          }
        }
      }
      if (p == 0) __syncthreads();
    }
    if (g.c_amax) amax_fold_wg(mx, g.c_amax, smem);
  }
}

// Waits of a stage that loaded the tiles of the stage after next: first for
// this lane's loads of the next stage and the scale words loaded at the start
// of this one (the KB_VM_TILES tile loads issued after them may stay in
// flight), later for its LDS writes before a plain s_barrier (a
// __syncthreads() would also wait for the loads in flight).  LDS reads of
// this stage have all been consumed by its MFMAs by then.
__device__ __forceinline__ void wait_vm_ahead() { asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); }
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One dword from global memory into a register, as inline assembly: the
// compiler does not track it, and the stage's explicit waits cover it.
__device__ __forceinline__ float load_word_untracked(const float* p) {
  float v;
  asm volatile("global_load_dword %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}

template <bool A2D, bool B2D, bool OUT_BF16>
__global__ __launch_bounds__(NTHR, 1) void gemm_blk_kernel(GemmArgs g) {
  static_assert(KB_VM_TILES == 12, "wait_vm_ahead counts 12 tile loads per stage");
  __shared__ __align__(16) uint8_t smem[KB_SMEM];

  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = w >> 1, wn = w & 1;
  const int lr = lane & 31, lg = lane >> 5;
  int tm, tn;
  tile_of(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * KB_BN;
  const int nk = g.K / 128;

  auto tA = [&](int s) { return smem + s * KB_STAGE; };
  auto tB = [&](int s) { return smem + s * KB_STAGE + TILEB; };
  auto ringA = [&](int s) { return (float*)(smem + KB_RING + s * KB_SLOT); };
  auto ringB = [&](int s) { return (float*)(smem + KB_RING + s * KB_SLOT + BM * 4); };

  Direct da;
  Direct4 db;
  direct_init(da, g.A, g.lda, m0, g.M, w);
  direct4_init(db, g.B, g.ldb, n0, g.N, w);
  auto issue_tile = [&](int kt, int v) {     // tile load v (of 12) of stage kt: A 0-7, B 8-11
    const int s = kt % KB_NSTAGE;
    if (v < 8) direct_item(da, kt, tA(s), w, v);
    else direct4_item(db, kt, tB(s), w, v - 8);
  };

  // Scale rows go through registers: lane (w, l) owns a_scale of tile row
  // 64 w + l and b_scale of tile row 64 (w & 1) + l; the words of stage k + 1
  // are loaded at the start of stage k and written into the LDS ring at its
  // end (waves 2-3 write their b_scale copy into the slot's sink).  Loads,
  // ring writes and ring reads are inline assembly with explicit waits: as
  // plain accesses the compiler cannot tell them apart from the tile loads
  // in flight and makes each wait for all of them.
  const int sstride = g.K / 128;
  int ra = m0 + 64 * w + lane, rb = n0 + 64 * (w & 1) + lane;
  ra = ra < g.M ? ra : g.M - 1;
  rb = rb < g.N ? rb : g.N - 1;
  const float* pa = (const float*)g.a_scale + (int64_t)(A2D ? ra / 128 : ra) * sstride;
  const float* pb = (const float*)g.b_scale + (int64_t)(B2D ? rb / 128 : rb) * sstride;
  auto put_scales = [&](int kt, float a, float b) {
    typedef __attribute__((address_space(3))) float* lds_f32_w;
    const int r = kt % KB_NSLOT;
    const lds_f32_w pa_ = (lds_f32_w)(ringA(r) + 64 * w + lane);
    const lds_f32_w pb_ = (lds_f32_w)(ringB(r) + (w < 2 ? 0 : KB_BN) + 64 * (w & 1) + lane);
    asm volatile("ds_write_b32 %0, %1" ::"v"(pa_), "v"(a) : "memory");
    asm volatile("ds_write_b32 %0, %1" ::"v"(pb_), "v"(b) : "memory");
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const uint32_t lb = (uint32_t)(lr * 128 + ((lg ^ swz_key(lr)) << 4));
  // B rows 64 wn + 32 j + lr have key(lr) ^ 2 j ^ 4 wn
  const uint32_t bx = (uint32_t)(wn << 6);

  // Operands of the current stage, carried across stages: B fragments of the
  // wave's two column tiles, A fragments of the current row tile, and the
  // raw scale words of the stage (read by inline assembly): a_scale of the
  // lane's row in each row tile, and b_scale -- one word for 128x128 weight
  // blocks, else the lane's 16 columns of each column tile.
  i32x8 fb[2][2], fa[2][2];
  uint32_t asw[4];
  i32x4 bsw[2][4];
  float fac[4] = {};     // per row tile: a_scale (times the weight scale for 128x128 blocks)
  float bsv[2][16] = {}; // 1x128 B blocks: b_scale of the lane's columns
  typedef __attribute__((address_space(3))) const float* lds_f32_p;
  auto read_fb = [&](int kt, int j) {
    const uint8_t* lbq = tB(kt % KB_NSTAGE) + wn * 8192;
#pragma unroll
    for (int h = 0; h < 2; ++h) fb[j][h] = read2(lbq + j * 4096, lb, ((uint32_t)(((4 * h) ^ (2 * j)) << 4)) ^ bx);
  };
  auto read_fa = [&](int kt, int i) {       // into fa[i & 1]
    const uint8_t* la = tA(kt % KB_NSTAGE) + wm * 16384;
#pragma unroll
    for (int h = 0; h < 2; ++h) fa[i & 1][h] = read2(la + i * 4096, lb, (uint32_t)(((4 * h) ^ (2 * i)) << 4));
  };
  auto load_scales = [&](int kt) {
    const lds_f32_p pa_ = (lds_f32_p)(ringA(kt % KB_NSLOT) + wm * 128 + lr);
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(asw[i]) : "v"(pa_), "i"(128 * i));
    if (B2D) {
      const lds_f32_p pb_ = (lds_f32_p)ringB(kt % KB_NSLOT);
      asm volatile("ds_read_b32 %0, %1" : "=v"(bsw[0][0].x) : "v"(pb_));
    } else {
      const lds_f32_p pb_ = (lds_f32_p)(ringB(kt % KB_NSLOT) + wn * 64 + 4 * lg);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(bsw[j][q]) : "v"(pb_), "i"(128 * j + 32 * q));
    }
  };
  // Wait for the scale reads (the wait names their results as operands, so
  // nothing that uses them is scheduled before it) and form the factors.
  auto finish_scales = [&]() {
    if (B2D) {
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(asw[0]), "+v"(asw[1]), "+v"(asw[2]), "+v"(asw[3]), "+v"(bsw[0][0].x)::"memory");
      const float bs = __uint_as_float(bsw[0][0].x);
#pragma unroll
      for (int i = 0; i < 4; ++i) fac[i] = __uint_as_float(asw[i]) * bs;
    } else {
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(asw[0]), "+v"(asw[1]), "+v"(asw[2]), "+v"(asw[3]), "+v"(bsw[0][0]), "+v"(bsw[0][1]),
                     "+v"(bsw[0][2]), "+v"(bsw[0][3]), "+v"(bsw[1][0]), "+v"(bsw[1][1]), "+v"(bsw[1][2]),
                     "+v"(bsw[1][3])::"memory");
#pragma unroll
      for (int i = 0; i < 4; ++i) fac[i] = __uint_as_float(asw[i]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 v = __builtin_bit_cast(float4, bsw[j][q]);
          bsv[j][4 * q] = v.x;
          bsv[j][4 * q + 1] = v.y;
          bsv[j][4 * q + 2] = v.z;
          bsv[j][4 * q + 3] = v.w;
        }
    }
  };

  // Prologue: scale words and tiles of stage 0, tiles of stage 1, then the
  // operands of stage 0.
  {
    const float a0 = pa[0], b0 = pb[0];
#pragma unroll
    for (int v = 0; v < KB_VM_TILES; ++v) issue_tile(0, v);
    if (nk > 1) {
#pragma unroll
      for (int v = 0; v < KB_VM_TILES; ++v) issue_tile(1, v);
    }
    put_scales(0, a0, b0);
    if (nk > 1) wait_vm_ahead();
    else wait_vm0();
    barrier_lds();
    read_fb(0, 0);
    read_fb(0, 1);
    read_fa(0, 0);
    load_scales(0);
  }

  // Partial products of the two tiles in flight; tile 7 of a stage is
  // folded during tile 0 of the next (zeros before the first stage).
  f32x16 part[2] = {};
  // fold values r0 .. r0 + 7 of tile tt with the current stage's scales
  auto fold8 = [&](int tt, int r0) {
    const int i = tt >> 1, j = tt & 1;
#pragma unroll
    for (int r = r0; r < r0 + 8; ++r)
      acc[i][j][r] = __builtin_fmaf(part[tt & 1][r], B2D ? fac[i] : fac[i] * bsv[j][r], acc[i][j][r]);
  };

  // One K stage.  MORE: stage kt + 2 exists and its tiles are loaded during
  // tiles 0-5 of this one; NEXT: stage kt + 1 exists (its scale words are
  // loaded here).  Tiles t = (i, j) = (t / 2, t % 2): tile t multiplies into
  // part[t % 2] while tile t - 1 is folded, acc += part * a_scale[m] *
  // b_scale[n]; tile 0 folds the previous stage's tile 7 before this
  // stage's scales replace that stage's.  A fragments of row tile i + 1 are
  // read into the other buffer once tile (i, 0) has issued.  After tile 5
  // every wave waits for the next stage's data and meets at a barrier (this
  // stage's tile buffer is no longer read by then), so tiles 6-7 read the
  // next stage's first operands as their registers free up, and the next
  // stage starts without an LDS round trip.  The last two stages are peeled
  // so that every stage is straight-line code and the fenced schedule holds.
  auto stage = [&](int kt, auto more_c, auto next_c) {
    constexpr bool MORE = decltype(more_c)::value;
    constexpr bool NEXT = decltype(next_c)::value;
    float a_nx = 0.0f, b_nx = 0.0f;
    if (NEXT) {
      a_nx = load_word_untracked(pa + kt + 1);
      b_nx = load_word_untracked(pb + kt + 1);
    }
    const f32x16 zero = {};
    // Each MFMA is followed by half a fold of the previous tile, so the
    // vector unit works while the matrix core does and the second MFMA of a
    // tile (which accumulates onto the first) finds the first one done.
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const int i = tt >> 1, j = tt & 1;
      // transposed tile: B rows are the instruction's rows, A rows its columns
      part[tt & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j][0], fa[i & 1][0], zero, 0, 0, 0, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      fold8((tt + 7) & 7, 0);
      if (MORE && tt < 6) issue_tile(kt + 2, 2 * tt);
      __builtin_amdgcn_sched_barrier(0);
      part[tt & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j][1], fa[i & 1][1], part[tt & 1], 0, 0, 0, 0,
                                                                     0, 0);
      __builtin_amdgcn_sched_barrier(0);
      fold8((tt + 7) & 7, 8);
      if (tt == 0) finish_scales();
      if (j == 0 && i < 3) read_fa(kt, i + 1);     // the other buffer: row tile i - 1 is done
      if (MORE && tt < 6) issue_tile(kt + 2, 2 * tt + 1);
      if (tt == 5 && NEXT) {
        if (MORE) wait_vm_ahead();
        else wait_vm0();
        put_scales(kt + 1, a_nx, b_nx);
        barrier_lds();
      }
      if (tt == 6 && NEXT) {                       // fb[0] is free once tile (3, 0) has issued, fa[0]
        read_fb(kt + 1, 0);                        // after row tile 2
        read_fa(kt + 1, 0);
      }
      if (tt == 7 && NEXT) read_fb(kt + 1, 1);     // fb[1] is free after tile (3, 1)
      __builtin_amdgcn_sched_barrier(0);
    }
    if (NEXT) load_scales(kt + 1);                 // fac / bsv still hold this stage's scales
  };
  using T_ = std::integral_constant<bool, true>;
  using F_ = std::integral_constant<bool, false>;
  for (int kt = 0; kt < nk - 2; ++kt) stage(kt, T_{}, T_{});
  if (nk >= 2) stage(nk - 2, F_{}, T_{});
  stage(nk - 1, F_{}, F_{});
  fold8(7, 0);
  fold8(7, 8);
  __syncthreads();                                   // the epilogue reuses the tile buffers
  store_blk<OUT_BF16>(acc, g, smem, m0, n0, w, wm, wn, lane);
}

gemm_fn blk_kernel_for(bool a2d, bool b2d, bool bf16_out) {
  if (a2d) {   // 128x128 blocks on A come with 128x128 blocks on B
    return bf16_out ? gemm_blk_kernel<true, true, true> : gemm_blk_kernel<true, true, false>;
  }
  if (b2d) return bf16_out ? gemm_blk_kernel<false, true, true> : gemm_blk_kernel<false, true, false>;
  return bf16_out ? gemm_blk_kernel<false, false, true> : gemm_blk_kernel<false, false, false>;
}

}  // namespace pbs
