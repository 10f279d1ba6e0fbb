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
// per output value and block.  Per wave and K block that is 16 MFMAs (1024
// matrix-core cycles) against 128 FMAs (512 vector cycles), plus 128 scale
// products for 1x128 B blocks.  The fold reads what the matrix core just
// wrote, so one wave alone leaves the matrix core idle whenever its
// instruction stream waits on that dependency, an LDS read or a barrier.
//
// So every SIMD runs two waves: a 256 x 256 output tile per workgroup, 8
// waves of 128 x 64 (2 along M x 4 along N), and while one wave folds or
// waits the other's MFMAs run.  Each wave keeps everything the fold touches
// in VGPRs -- 128 accumulators per lane, and the MFMAs write their partial
// products to VGPRs (this file is built with -amdgpu-mfma-vgpr-form) -- in
// the 256 registers two waves per SIMD leave it.  The fold of tile t-1 runs
// while tile t multiplies.
//
// Staging: two LDS stage buffers of 64 KB (A and B, 256 rows x 128 B each,
// swizzled as in the other GEMMs) and a 2-deep scale-row ring, all filled by
// LDS-DMA.  The loads of stage k+2 are issued in the last two tiles of stage
// k, as soon as every wave is done reading stage k's buffer, and waited for
// in the middle of stage k+1.  One barrier per stage.
#include "device.hpp"
#include "gemm_common.hpp"
#include "host.hpp"

#include <type_traits>

namespace pbs {

constexpr int KB_THR = BLK_THR;                     // 8 waves per workgroup
constexpr int KB_NW = KB_THR / 64;
constexpr int KB_BN = BLK_BN;                      // output columns per workgroup
constexpr int KB_STAGE = 2 * TILEB;                // A and B: 64 KB per stage
constexpr int KB_NSTAGE = 2;
constexpr int KB_RING = KB_NSTAGE * KB_STAGE;      // scale ring after the stage buffers
constexpr int KB_NSLOT = 2;
constexpr int KB_SLOT = (BM + KB_BN) * 4;          // a_scale[256], b_scale[256]
constexpr int KB_STG_BF16 = 2 * KB_BN + 16;        // epilogue staging pitch in bytes, bf16 (256 rows)
constexpr int KB_STG_F32 = 4 * KB_BN + 16;         // fp32 (128 rows a pass)
constexpr int KB_SMEM = cmax(KB_RING + KB_NSLOT * KB_SLOT, cmax(BM * KB_STG_BF16, 128 * KB_STG_F32));
static_assert(KB_SMEM <= 160 * 1024, "LDS");

// Tile loads: 256 rows, 4 loads per lane; load i of wave w (0-7) fills rows
// 32 w + 8 i .. + 7; lane l owns row 32 w + 8 i + l / 8, physical chunk l % 8
// (the logical chunk that the swizzle places there).
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
                                          int wm, int wn, int lane) {
  const int t = threadIdx.x;
  const int lr = lane & 31, lg = lane >> 5;
  const bool full = (m0 + BM <= g.M) && (n0 + KB_BN <= g.N);
  uint32_t mx = 0;
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
    const int ch = t & 31;                           // 16-byte chunk of a 512-byte row
#pragma unroll 4
    for (int it = 0; it < 16; ++it) {
      const int s = 16 * it + (t >> 5);
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
  } else {
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
      const int ch = t & 63;                         // 16-byte chunk of a 1 KB row
#pragma unroll 4
      for (int it = 0; it < 16; ++it) {
        const int s = 8 * it + (t >> 6);
        const uint4 val = *(const uint4*)(smem + s * KB_STG_F32 + ch * 16);
        const int grow = m0 + 128 * p + s, gcol = n0 + ch * 4;
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
  }
  if (g.c_amax) amax_fold_wg<KB_NW>(mx, g.c_amax, smem);
}

// The wait in the middle of a stage for this lane's loads of the next stage
// (nothing else is in flight then), and for its LDS accesses before a plain
// s_barrier (a __syncthreads() would do the same here, but says less).
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <bool A2D, bool B2D, bool OUT_BF16>
__global__ __launch_bounds__(KB_THR, 1) void gemm_blk_kernel(GemmArgs g) {
  __shared__ __align__(16) uint8_t smem[KB_SMEM];

  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = w >> 2, wn = w & 3;
  const int lr = lane & 31, lg = lane >> 5;
  int tm, tn;
  tile_of(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * KB_BN;
  const int nk = g.K / 128;

  auto tA = [&](int s) { return smem + (s & 1) * KB_STAGE; };
  auto tB = [&](int s) { return smem + (s & 1) * KB_STAGE + TILEB; };
  auto ringA = [&](int s) { return (float*)(smem + KB_RING + (s & 1) * KB_SLOT); };
  auto ringB = [&](int s) { return (float*)(smem + KB_RING + (s & 1) * KB_SLOT + BM * 4); };

  Direct4 da, db;
  direct4_init(da, g.A, g.lda, m0, g.M, w);
  direct4_init(db, g.B, g.ldb, n0, g.N, w);
  // Scale rows go into the ring by LDS-DMA like the tiles: lane (w, l) of
  // waves 0-3 loads the a_scale word of tile row 64 w + l, of waves 4-7 the
  // b_scale word of tile row 64 (w - 4) + l.
  const int sstride = g.K / 128;
  const float* ps;
  {
    const bool on_a = w < 4;
    int r = on_a ? m0 + 64 * w + lane : n0 + 64 * (w - 4) + lane;
    const int lim = on_a ? g.M : g.N;
    r = r < lim ? r : lim - 1;
    const bool twod = on_a ? A2D : B2D;
    ps = (const float*)(on_a ? g.a_scale : g.b_scale) + (int64_t)(twod ? r / 128 : r) * sstride;
  }
  // load v (of 9) of stage kt: A tiles 0-3, B tiles 4-7, the scale word 8
  auto issue_item = [&](int kt, int v) {
    if (v < 4) {
      direct4_item(da, kt, tA(kt), w, v);
    } else if (v < 8) {
      direct4_item(db, kt, tB(kt), w, v - 4);
    } else {
      __builtin_amdgcn_global_load_lds(ps + kt, (lds_ptr_t)(ringA(kt) + 64 * w), 4, 0, 0);
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const uint32_t lb = (uint32_t)(lr * 128 + ((lg ^ swz_key(lr)) << 4));
  // B rows 64 wn + 32 j + lr have key(lr) ^ 2 j ^ 4 (wn & 1)
  const uint32_t bx = (uint32_t)((wn & 1) << 6);

  using T_ = std::integral_constant<bool, true>;
  using F_ = std::integral_constant<bool, false>;
  uint32_t asw[4];       // a_scale words of the lane's row in each row tile (fp32 bits)
  float fac[4] = {};     // per row tile: a_scale (times the weight scale for 128x128 blocks)
  auto read_asw = [&](int kt) {
    const float* qa = ringA(kt) + wm * 128 + lr;
#pragma unroll
    for (int i = 0; i < 4; ++i) asw[i] = __float_as_uint(qa[32 * i]);
  };
  // The prologue issues the loads of stages 0 and 1 and waits for stage 0
  // with stage 1's 9 loads in flight: a counted wait, right only while the
  // kernel does not spill (spill traffic is counted too); the static check
  // of this file holds every variant to that.

  if constexpr (B2D) {
    // Operands of the current stage, carried across stages: B fragments of
    // the wave's two column tiles, A fragments of the current row tile, the
    // a_scale words and the one b_scale word of the wave's 64 columns (they
    // lie in one 128x128 block).
    i32x8 fb[2][2], fa[2];
    uint32_t bsw = 0;
    auto read_fb = [&](int kt, int j) {
      const uint8_t* lbq = tB(kt) + wn * 8192;
#pragma unroll
      for (int h = 0; h < 2; ++h) fb[j][h] = read2(lbq + j * 4096, lb, ((uint32_t)(((4 * h) ^ (2 * j)) << 4)) ^ bx);
    };
    auto read_fa = [&](int kt, int i) {
      const uint8_t* la = tA(kt) + wm * 16384;
#pragma unroll
      for (int h = 0; h < 2; ++h) fa[h] = read2(la + i * 4096, lb, (uint32_t)(((4 * h) ^ (2 * i)) << 4));
    };
    auto load_scales = [&](int kt) {
      read_asw(kt);
      bsw = __float_as_uint(ringB(kt)[64 * wn]);
    };
    auto finish_scales = [&]() {
      const float bs = __uint_as_float(bsw);
#pragma unroll
      for (int i = 0; i < 4; ++i) fac[i] = __uint_as_float(asw[i]) * bs;
    };

    {
#pragma unroll
      for (int v = 0; v < 9; ++v) issue_item(0, v);
      if (nk > 1) {
#pragma unroll
        for (int v = 0; v < 9; ++v) issue_item(1, v);
        asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
      } else {
        wait_vm0();
      }
      barrier_lds();
      read_fb(0, 0);
      read_fb(0, 1);
      read_fa(0, 0);
      load_scales(0);
    }

    // Partial products of the two tiles in flight: tile t multiplies while
    // tile t - 1 is folded, and tile 7 of a stage is folded during tile 0 of
    // the next (zeros before the first stage).
    f32x16 part[2] = {};
    auto fold8 = [&](int tt, int r0) {           // values r0 .. r0 + 7 of tile tt
      const int i = tt >> 1, j = tt & 1;
#pragma unroll
      for (int r = r0; r < r0 + 8; ++r) acc[i][j][r] = __builtin_fmaf(part[tt & 1][r], fac[i], acc[i][j][r]);
    };

    // One K stage.  ISSUE: stage kt + 2 exists and its loads are issued in
    // tiles 6-7 of this one, into this stage's buffer and ring slot; NEXT:
    // stage kt + 1 exists.  Tiles t = (i, j) = (t / 2, t % 2): tile t
    // multiplies into part[t % 2] while tile t - 1 is folded, acc += part *
    // a_scale[m] * b_scale[n]; tile 0 folds the previous stage's tile 7
    // before this stage's scales replace that stage's.  A fragments of row
    // tile i + 1 are read once tile (i, 1) has issued (the other wave of the
    // SIMD covers the LDS latency).  After tile 5 every wave waits for the
    // next stage's data and meets at a barrier (this stage's buffer is no
    // longer read by then), so tiles 6-7 read the next stage's first operands
    // as their registers free up and refill this stage's buffer, and the next
    // stage starts without an LDS round trip.  The last stages are peeled so
    // that every stage is straight-line code and the fenced schedule holds.
    auto stage = [&](int kt, auto issue_c, auto next_c) {
      constexpr bool ISSUE = decltype(issue_c)::value;
      constexpr bool NEXT = decltype(next_c)::value;
      const f32x16 zero = {};
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const int i = tt >> 1, j = tt & 1;
        // transposed tile: B rows are the instruction's rows, A rows its columns
        part[tt & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j][0], fa[0], zero, 0, 0, 0, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        fold8((tt + 7) & 7, 0);
        if (ISSUE && tt == 6) {
#pragma unroll
          for (int v = 0; v < 3; ++v) issue_item(kt + 2, v);
        }
        if (ISSUE && tt == 7) {
#pragma unroll
          for (int v = 5; v < 7; ++v) issue_item(kt + 2, v);
        }
        __builtin_amdgcn_sched_barrier(0);
        part[tt & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j][1], fa[1], part[tt & 1], 0, 0, 0, 0, 0,
                                                                       0);
        __builtin_amdgcn_sched_barrier(0);
        fold8((tt + 7) & 7, 8);
        if (tt == 0) finish_scales();              // the previous stage's scales are done with
        if (j == 1 && i < 3) read_fa(kt, i + 1);   // row tile i is done
        if (ISSUE && tt == 6) {
#pragma unroll
          for (int v = 3; v < 5; ++v) issue_item(kt + 2, v);
        }
        if (ISSUE && tt == 7) {
#pragma unroll
          for (int v = 7; v < 9; ++v) issue_item(kt + 2, v);
        }
        if (tt == 5 && NEXT) {
          wait_vm0();
          barrier_lds();
        }
        if (tt == 6 && NEXT) read_fb(kt + 1, 0);   // fb[0] is free once tile (3, 0) has issued
        if (tt == 7 && NEXT) {                     // fa, fb[1] are free after tile (3, 1)
          read_fb(kt + 1, 1);
          read_fa(kt + 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (NEXT) load_scales(kt + 1);               // fac still holds this stage's scales
    };
    for (int kt = 0; kt < nk - 2; ++kt) stage(kt, T_{}, T_{});
    if (nk >= 2) stage(nk - 2, F_{}, T_{});
    stage(nk - 1, F_{}, F_{});
    fold8(7, 0);
    fold8(7, 8);
  } else {
    // 1x128 B blocks: the lane's 16 columns of a column tile have 16
    // different b_scale words.  Tiles go column tile by column tile, t =
    // (i, j) = (t % 4, t / 4), so that only one column tile's words are held
    // (16 registers rather than 32, which keeps the wave within its 256
    // without spilling), at the cost of reading the A fragments twice per
    // stage; each tile's partial products are folded right after its MFMAs
    // (the SIMD's other wave covers the wait), the A fragments of the next
    // tile are read into the other of two buffers meanwhile.
    i32x8 gb[2], ga[2][2];
    i32x4 bw[4];
    auto read_gb = [&](int kt, int j) {
      const uint8_t* lbq = tB(kt) + wn * 8192;
#pragma unroll
      for (int h = 0; h < 2; ++h) gb[h] = read2(lbq + j * 4096, lb, ((uint32_t)(((4 * h) ^ (2 * j)) << 4)) ^ bx);
    };
    auto read_ga = [&](int kt, int i, int slot) {
      const uint8_t* la = tA(kt) + wm * 16384;
#pragma unroll
      for (int h = 0; h < 2; ++h) ga[slot][h] = read2(la + i * 4096, lb, (uint32_t)(((4 * h) ^ (2 * i)) << 4));
    };
    auto read_bw = [&](int kt, int j) {
      const float* qb = ringB(kt) + wn * 64 + 32 * j + 4 * lg;
#pragma unroll
      for (int q = 0; q < 4; ++q) bw[q] = *(const i32x4*)(qb + 8 * q);
    };

    {
#pragma unroll
      for (int v = 0; v < 9; ++v) issue_item(0, v);
      if (nk > 1) {
#pragma unroll
        for (int v = 0; v < 9; ++v) issue_item(1, v);
        asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
      } else {
        wait_vm0();
      }
      barrier_lds();
      read_gb(0, 0);
      read_ga(0, 0, 0);
      read_bw(0, 0);
      read_asw(0);
    }

    // One K stage, ISSUE / NEXT as for 128x128 blocks.  After tile 6 (whose
    // A read for tile 7 is this stage's last read of its buffer) every wave
    // waits for the next stage's data and meets at a barrier; tiles 6-7 then
    // refill this stage's buffer and tile 7 reads the next stage's first
    // operands and scale words.
    auto stage = [&](int kt, auto issue_c, auto next_c) {
      constexpr bool ISSUE = decltype(issue_c)::value;
      constexpr bool NEXT = decltype(next_c)::value;
      const f32x16 zero = {};
#pragma unroll
      for (int i = 0; i < 4; ++i) fac[i] = __uint_as_float(asw[i]);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int i = t & 3, j = t >> 2, sl = t & 1;
        f32x16 part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(gb[0], ga[sl][0], zero, 0, 0, 0, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(gb[1], ga[sl][1], part, 0, 0, 0, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (t < 7) read_ga(kt, (t + 1) & 3, sl ^ 1);   // the other buffer: tile t - 1 is done
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc[i][j][r] = __builtin_fmaf(part[r] * __builtin_bit_cast(float4, bw[r >> 2])[r & 3], fac[i], acc[i][j][r]);
        if (t == 3) {                               // column tile 0 is done
          read_gb(kt, 1);
          read_bw(kt, 1);
        }
        if (t == 6 && NEXT) {
          wait_vm0();
          barrier_lds();
        }
        if (ISSUE && t == 6) {
#pragma unroll
          for (int v = 0; v < 5; ++v) issue_item(kt + 2, v);
        }
        if (ISSUE && t == 7) {
#pragma unroll
          for (int v = 5; v < 9; ++v) issue_item(kt + 2, v);
        }
        if (t == 7 && NEXT) {
          read_gb(kt + 1, 0);
          read_ga(kt + 1, 0, 0);
          read_bw(kt + 1, 0);
          read_asw(kt + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    for (int kt = 0; kt < nk - 2; ++kt) stage(kt, T_{}, T_{});
    if (nk >= 2) stage(nk - 2, F_{}, T_{});
    stage(nk - 1, F_{}, F_{});
  }
  __syncthreads();                                   // the epilogue reuses the tile buffers
  store_blk<OUT_BF16>(acc, g, smem, m0, n0, wm, wn, lane);
}

gemm_fn blk_kernel_for(bool a2d, bool b2d, bool bf16_out) {
  if (a2d) {   // 128x128 blocks on A come with 128x128 blocks on B
    return bf16_out ? gemm_blk_kernel<true, true, true> : gemm_blk_kernel<true, true, false>;
  }
  if (b2d) return bf16_out ? gemm_blk_kernel<false, true, true> : gemm_blk_kernel<false, true, false>;
  return bf16_out ? gemm_blk_kernel<false, false, true> : gemm_blk_kernel<false, false, false>;
}

}  // namespace pbs
