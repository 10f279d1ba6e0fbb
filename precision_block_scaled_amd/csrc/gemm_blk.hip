// Sub-channel FP8 GEMM: 1x128 blocks for activations and gradients, 128x128
// (Fprop / Dgrad weights) or 1x128 (Wgrad) blocks for the other operand
// ("Faster training throughput in FP8 precision with NVIDIA NeMo",
// "Scaling recipe granularity").
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
constexpr int KB_NSLOT = 2;
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

template <bool OUT_BF16>
__device__ __forceinline__ void store_blk(f32x16 (&acc)[4][2], const GemmArgs& g, uint8_t* smem, int m0, int n0,
                                          int w, int wm, int wn, int lane) {
  const int lr = lane & 31, lg = lane >> 5;
  const bool full = (m0 + BM <= g.M) && (n0 + KB_BN <= g.N);
  if constexpr (OUT_BF16) {
    // lanes lr and lr ^ 1 swap halves so each writes two rows of a column pair
    const int par = lr & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1];
          const float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
          const uint32_t own = par ? pk_bf16(v2, v3) : pk_bf16(v0, v1);
          const uint32_t snd = par ? pk_bf16(v0, v1) : pk_bf16(v2, v3);
          const uint32_t rcv = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)snd, 0xB1, 0xF, 0xF, false);
          const uint32_t lo = par ? rcv : own, hi = par ? own : rcv;
          const int row = wm * 128 + 32 * i + 8 * q + 4 * lg + 2 * par;
          const int colb = (wn * 64 + 32 * j + (lr & ~1)) * 2;
          *(uint32_t*)(smem + row * KB_STG_BF16 + colb) = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
          *(uint32_t*)(smem + (row + 1) * KB_STG_BF16 + colb) = __builtin_amdgcn_perm(hi, lo, 0x07060302u);
        }
    __syncthreads();
    const int ch = lane & 15;
#pragma unroll 4
    for (int it = 0; it < 16; ++it) {
      const int s = 64 * w + 4 * it + (lane >> 4);
      const uint4 val = *(const uint4*)(smem + s * KB_STG_BF16 + ch * 16);
      const int grow = m0 + s, gcol = n0 + ch * 8;
      if (full || (grow < g.M && gcol < g.N))
        *(uint4*)((uint16_t*)g.C + (int64_t)grow * g.ldc + gcol) = val;
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
            for (int r = 0; r < 16; ++r) {
              const int row = 32 * i + 8 * (r >> 2) + 4 * lg + (r & 3);
              const int col = wn * 64 + 32 * j + lr;
              *(float*)(smem + row * KB_STG_F32 + col * 4) = acc[i][j][r];
            }
      }
      __syncthreads();
#pragma unroll 4
      for (int it = 0; it < 16; ++it) {
        const int s = 32 * w + 2 * it + (lane >> 5);
        const uint4 val = *(const uint4*)(smem + s * KB_STG_F32 + (lane & 31) * 16);
        const int grow = m0 + 128 * p + s, gcol = n0 + (lane & 31) * 4;
        if (full || (grow < g.M && gcol < g.N)) *(uint4*)((float*)g.C + (int64_t)grow * g.ldc + gcol) = val;
      }
      if (p == 0) __syncthreads();
    }
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

template <bool B2D, bool OUT_BF16>
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
  const float* pa = (const float*)g.a_scale + (int64_t)ra * sstride;
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

  {
    const float a0 = pa[0], b0 = pb[0];
#pragma unroll
    for (int v = 0; v < KB_VM_TILES; ++v) issue_tile(0, v);
    if (nk > 1) {
#pragma unroll
      for (int v = 0; v < KB_VM_TILES; ++v) issue_tile(1, v);
    }
    put_scales(0, a0, b0);
    wait_vm0();
    __syncthreads();
  }

  // One K stage.  MORE: stage kt + 2 exists and its tiles are loaded during
  // this one; NEXT: stage kt + 1 exists (its scale words are loaded here).
  // The last two stages are peeled so that every stage is straight-line code
  // and the fenced schedule holds.
  auto stage = [&](int kt, auto more_c, auto next_c) {
    constexpr bool MORE = decltype(more_c)::value;
    constexpr bool NEXT = decltype(next_c)::value;
    const int s = kt % KB_NSTAGE;
    const uint8_t* la = tA(s) + wm * 16384;
    const uint8_t* lbq = tB(s) + wn * 8192;
    const float* sca = ringA(kt % KB_NSLOT) + wm * 128 + lg * 4;
    const float* scb = ringB(kt % KB_NSLOT) + wn * 64 + lr;
    float a_nx = 0.0f, b_nx = 0.0f;
    if (NEXT) {
      a_nx = load_word_untracked(pa + kt + 1);
      b_nx = load_word_untracked(pb + kt + 1);
    }

    i32x8 fb[2][2], fa[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) fb[j][h] = read2(lbq + j * 4096, lb, ((uint32_t)(((4 * h) ^ (2 * j)) << 4)) ^ bx);
#pragma unroll
    for (int h = 0; h < 2; ++h) fa[h] = read2(la, lb, (uint32_t)((4 * h) << 4));
    float sbv[2];
    sbv[0] = scb[0];
    sbv[1] = B2D ? sbv[0] : scb[32];
    // scale factors of one row tile: a_scale of the lane's 16 rows (4
    // consecutive rows per 16-byte read), times the weight scale for 128x128
    // blocks
    float fac[16];
    i32x4 facw[4];
    auto load_fac = [&](int i) {
      typedef __attribute__((address_space(3))) const float* lds_f32_p;
      const lds_f32_p p = (lds_f32_p)(sca + 32 * i);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(facw[q]) : "v"(p), "i"(32 * q));
    };
    // after load_fac: wait for the reads (the wait names their results as
    // operands, so nothing that uses them is scheduled before it), then fold
    // in the weight scale of 128x128 blocks
    auto finish_fac = [&]() {
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(facw[0]), "+v"(facw[1]), "+v"(facw[2]), "+v"(facw[3]) :: "memory");
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = __builtin_bit_cast(float4, facw[q]);
        fac[4 * q] = v.x;
        fac[4 * q + 1] = v.y;
        fac[4 * q + 2] = v.z;
        fac[4 * q + 3] = v.w;
      }
      if (B2D) {
#pragma unroll
        for (int r = 0; r < 16; ++r) fac[r] *= sbv[0];
      }
    };
    load_fac(0);
    finish_fac();

    // Tiles t = (i, j) = (t / 2, t % 2).  Tile t multiplies into part[t % 2]
    // while tile t - 1 is folded.  A fragments of row tile i + 1 are read once
    // tile (i, 1) has issued; the scale factors of row tile i once tile
    // (i - 1, 1) is folded, one MFMA pair before their first use.
    f32x16 part[2];
    auto fold = [&](int tt) {
      const int j = tt & 1;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        acc[tt >> 1][j][r] = __builtin_fmaf(part[tt & 1][r], B2D ? fac[r] : fac[r] * sbv[j], acc[tt >> 1][j][r]);
    };
    const f32x16 zero = {};
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const int i = tt >> 1, j = tt & 1;
      part[tt & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[0], fb[j][0], zero, 0, 0, 0, 0, 0, 0);
      part[tt & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[1], fb[j][1], part[tt & 1], 0, 0, 0, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (j == 1 && i > 0) finish_fac();
      if (tt > 0) fold(tt - 1);
      if (j == 1 && i < 3) {
#pragma unroll
        for (int h = 0; h < 2; ++h) fa[h] = read2(la + (i + 1) * 4096, lb, (uint32_t)(((4 * h) ^ (2 * (i + 1))) << 4));
      }
      if (j == 0 && i > 0) load_fac(i);
      if (MORE) {
#pragma unroll
        for (int v = (KB_VM_TILES * tt) / 8; v < (KB_VM_TILES * (tt + 1)) / 8; ++v) issue_tile(kt + 2, v);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    fold(7);
    if (MORE) {
      wait_vm_ahead();
      put_scales(kt + 1, a_nx, b_nx);
      barrier_lds();
    } else {
      wait_vm0();
      if (NEXT) put_scales(kt + 1, a_nx, b_nx);
      __syncthreads();
    }
  };
  using T_ = std::integral_constant<bool, true>;
  using F_ = std::integral_constant<bool, false>;
  for (int kt = 0; kt < nk - 2; ++kt) stage(kt, T_{}, T_{});
  if (nk >= 2) stage(nk - 2, F_{}, T_{});
  stage(nk - 1, F_{}, F_{});
  store_blk<OUT_BF16>(acc, g, smem, m0, n0, w, wm, wn, lane);
}

gemm_fn blk_kernel_for(bool b2d, bool bf16_out) {
  if (b2d) return bf16_out ? gemm_blk_kernel<true, true> : gemm_blk_kernel<true, false>;
  return bf16_out ? gemm_blk_kernel<false, true> : gemm_blk_kernel<false, false>;
}

}  // namespace pbs
