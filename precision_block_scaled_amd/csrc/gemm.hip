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
//              natural-layout tensors, MN-contiguous; MN-contiguous tiles go
//              to LDS as stored and are transposed by the fragment reads
//              (ds_read_b64_tr_b16).
//  FP8 per-tensor  v_mfma_f32_32x32x64_f8f6f4 (format per operand: E4M3 or
//              E5M2), scales applied once in the epilogue.
//  FP8 1x128 / 128x128  gemm_blk.hip (the fp32 block scales are folded in
//              by the vector unit; that kernel keeps its accumulators in VGPRs).
//  MXFP8       v_mfma_scale_f32_32x32x64_f8f6f4: each K=64 step covers two
//              MX blocks; the two lanes that hold a row (or column) each
//              supply the E8M0 scale of one of its blocks, and the hardware
//              applies it to that block's 32 products.
//  FP8 1x128 / 128x128 with power-of-two scales  the MXFP8 kernel: a
//              128-long K stage is one block, and its scale word repeats the
//              block's E8M0 code in all four bytes, so the instruction applies
//              it to each 32-value step; the 128x128 weight blocks share one
//              scale row per 128 operand rows.
//  NVFP4       E2M1 x E4M3 block scale has up to 6 significant bits, more
//              than any 4-, 6- or 8-bit MFMA input holds, and the E4M3 scale
//              is no power of two, so it cannot ride on the instruction's
//              E8M0 scale either.  The scales are applied in registers: raw
//              E2M1 tiles sit in LDS and every wave decodes its operands
//              exactly into fp16 (E2M1 -> fp16 by conversion, times the block
//              scale by an exact fp16 multiply: the product needs <= 6 bits
//              and lies in [2^-10, 2688]) right before
//              v_mfma_f32_32x32x16_f16 (gemm_nvfp4_kernel).  The two fp32
//              tensor scales are applied in the epilogue.
//
// Tiling: 256 x 256 output tile per workgroup of 256 threads (4 waves in a
// 2 x 2 grid, 128 x 128 per wave = 4 x 4 MFMA 32x32 tiles, 256 fp32
// accumulators per lane).  Each K stage moves 128 bytes per operand row
// (64 bf16, 128 fp8, 256 E2M1): 32 KB per operand (16 KB for E2M1),
// double-buffered in LDS.  Operand tiles go global -> LDS directly
// (buffer_load_dwordx4 ... lds, no registers; NVFP4 tiles and scale rows
// global_load_lds), each lane fetching the 16-byte chunk whose
// XOR-swizzled LDS slot it owns; the swizzle makes the
// MFMA fragment reads (ds_read_b128) bank-conflict-free.  MN-major bf16
// tiles are read with the transposing ds_read_b64_tr_b16.  Workgroups are mapped to tiles
// so that each of the 8 XCDs (each with its own L2) works on a contiguous,
// row-grouped range of tiles.
#include "device.hpp"
#include "gemm_common.hpp"
#include "host.hpp"

#include <type_traits>

namespace pbs {

enum { OP_BF16 = 0, OP_FP8 = 2, OP_FP4 = 3 };               // what the MFMA consumes
enum { LD_KMAJOR = 0, LD_MNMAJOR = 1 };                      // how a tile reaches LDS
// SC_MXC: MX scales loaded in 16-byte chunks; SC_CHAN: one fp32 scale per row
// of A and of B, applied in the epilogue
enum { SC_NONE = 0, SC_TENSOR = 1, SC_MX = 2, SC_MXC = 3, SC_CHAN = 4 };

constexpr int BN = 256;
constexpr int SC_OFF = 4 * TILEB;       // scale-row ring after 2 stages x 2 operands
constexpr int SC_RING = 3;
constexpr int STG_BF16 = 544;           // epilogue staging row pitch, bf16 output (256 rows)
constexpr int STG_F32 = 1056;           // epilogue staging row pitch, fp32 output (128 rows a pass)
// scale dwords per row per stage: MXFP8 4 E8M0 bytes (128 values), MXFP4 8 (256)
constexpr int sc_dw(int op) { return op == OP_FP4 ? 2 : 1; }
// MX scale chunks: 16 bytes per row (4 stages of MXFP8, 2 of MXFP4), two
// slots per operand
constexpr int smem_bytes(int op, int sc) {
  return cmax(SC_OFF + (sc == SC_MXC ? 2 * 2 * BM * 16 : SC_RING * 2 * BM * 4 * sc_dw(op)),
              cmax(256 * STG_BF16, 128 * STG_F32));
}
constexpr int SMEM = smem_bytes(OP_FP8, SC_TENSOR);

// Instruction classes for __builtin_amdgcn_sched_group_barrier.
enum : int { SG_VALU = 0x002, SG_MFMA = 0x008, SG_VMEM = 0x010, SG_DSR = 0x100, SG_DSW = 0x200 };
#define PBS_SCHED(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)

// Dword q of DW per row per stage (MXFP4: 8 scale bytes per row and stage),
// into plane q of the ring slot (planes BM dwords apart).
template <int DW>
__device__ __forceinline__ void rowdw_issue_q(const RowDword& d, int kt, int q, uint32_t* ring_slot, int w) {
  __builtin_amdgcn_global_load_lds(d.p + (int64_t)kt * 4 * DW + 4 * q, (lds_ptr_t)(ring_slot + q * BM + 64 * w), 4,
                                   0, 0);
}

// MN-major bf16 (stored [K][MN], the Dgrad / Wgrad operands in natural
// layout): the stage's 64 K rows of the tile's 256 MN values (512 bytes)
// go to LDS as they are, rows K-indexed, with 16-byte chunk c of row k at
// k * 512 + ((c ^ 4 (k & 3)) << 4).  Load i (of 8) of wave w fills rows
// 2 q, 2 q + 1 (q = 8 w + i); lane l owns row 2 q + l / 32, physical chunk
// l % 32.  Chunks past the MN extent re-read the last valid chunk.  Each
// stage's 64 rows are one buffer resource (its base is scalar arithmetic),
// so a load takes the lane's 32-bit offset as it is.
struct MnDirect {
  const uint8_t* base;    // operand + mn0 * 2 (wave-uniform)
  int64_t kstep;          // bytes per K stage: 64 rows
  uint32_t off[8];
};

__device__ __forceinline__ void mn_direct_init(MnDirect& d, const uint8_t* p, int64_t ld, int mn0, int nmn, int w) {
  const int lane = threadIdx.x & 63;
  d.base = p + (int64_t)mn0 * 2;
  d.kstep = 64 * ld;
  const int lastc = (nmn - mn0 - 8) >> 3;     // last chunk of the tile with valid columns
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 2 * (8 * w + i) + (lane >> 5);
    int lc = (lane & 31) ^ (4 * (row & 3));
    lc = lc < lastc ? lc : lastc;
    d.off[i] = (uint32_t)row * (uint32_t)ld + (uint32_t)(lc << 4);
  }
}

__device__ __forceinline__ void mn_direct_item(const MnDirect& d, int kt, uint8_t* tile, int w, int i) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)(d.base + kt * d.kstep), (short)0, (int)d.kstep, BUF_RSRC_WORD3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(tile + (w * 8 + i) * 1024), 16, d.off[i], 0, 0, 0);
}

// Fragments of one half K-stage (64 of the 128 bytes of every LDS row): for
// each of the wave's 4 row tiles (A) and 4 column tiles (B), lane (lr, lg)
// holds 16-byte chunks 4h + lg (elements 0-3) and 4h + 2 + lg (elements
// 4-7) of its row.  For 8-bit operands the 8 dwords are one K=64 MFMA
// operand (see the layout note in the kernel); for 16-bit operands the two
// halves are the operands of two K=16 steps (chunks 2s + lg, s = 2h, 2h + 1).
//
// Address: row = 128 wm + 32 i + lr has key(row) = key(lr) ^ 2 i, so the
// physical chunk is (lg ^ key(lr)) ^ 4 h ^ 2 i (^ 2 for the upper half): one
// per-lane constant lb = 128 lr + ((lg ^ key(lr)) << 4), XOR-ed with a
// compile-time pattern.
struct Frags {
  i32x4 a[4][2], b[4][2];     // [tile][lower / upper 16 bytes]
};

// LDS reads of one operand for a half stage.  K-major: read d (of 8) is
// tile d / 2, part d % 2 (one ds_read_b128).  MN-major: read d (of 16) is
// tile d / 4, K=16 step s = (d / 2) % 2 of the half, 4-value quarter q = d % 2,
// one ds_read_b64_tr_b16: within each 16-lane group, lane j addresses 4
// consecutive MN values of K row 16 S + 8 lg + 4 q + j / 4 (S = 2 H + s), and
// the transposing read hands lane i the 4 K values of MN column i.  The
// per-lane part of that address is lm = (8 lg + j / 4) * 512 + 64 (j / 4) +
// 16 (2 h' + (j % 4) / 2) + 8 (j % 2) + 256 wm (h' = lr / 16, j = lr % 16);
// tile i XORs 64 i into it (the chunk swizzle 4 (k & 3) = 4 (j / 4)).
// One transposing read.  The compiler makes an LDS read wait for every
// LDS-DMA load in flight unless the read carries alias information; a
// restrict-qualified pointer gives it some, and the compiler then separates
// the read from the loads by their addresses, as it does for the plain
// ds_read_b128 of K-major tiles (the loads in flight fill the other stage
// buffer; the stage's own loads were waited for at the barrier).
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i16x4 read_tr16(const uint8_t* __restrict__ p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

template <int H, int LD>
__device__ __forceinline__ void op_read(i32x4 (&x)[4][2], int d, const uint8_t* base, uint32_t lb) {
  if (LD == LD_KMAJOR) {
    const int tile = d >> 1, part = d & 1;
    const uint32_t xo = (uint32_t)((((4 * H) ^ (2 * tile)) << 4) ^ (part << 5));
    x[tile][part] = *(const i32x4*)(base + tile * 4096 + (lb ^ xo));
  } else {
    const int tile = d >> 2, s = (d >> 1) & 1, q = d & 1;
    const int S = 2 * H + s;
    const i16x4 v = read_tr16(base + (16 * S + 4 * q) * 512 + (lb ^ (uint32_t)(64 * tile)));
    const int2 w2 = __builtin_bit_cast(int2, v);
    if (q == 0) {
      x[tile][s].x = w2.x;
      x[tile][s].y = w2.y;
    } else {
      x[tile][s].z = w2.x;
      x[tile][s].w = w2.y;
    }
  }
}

template <int LD>
constexpr int op_reads() { return LD == LD_KMAJOR ? 8 : 16; }

// LDS read d of a half stage: A's reads first, then B's.
template <int H, int LDA, int LDB>
__device__ __forceinline__ void frag_read(Frags& f, int d, const uint8_t* la, const uint8_t* lbp, uint32_t lba,
                                          uint32_t lbb) {
  if (d < op_reads<LDA>()) op_read<H, LDA>(f.a, d, la, lba);
  else op_read<H, LDB>(f.b, d - op_reads<LDA>(), lbp, lbb);
}

__device__ __forceinline__ i32x8 cat(const i32x4 (&p)[2]) {
  return __builtin_shufflevector(p[0], p[1], 0, 1, 2, 3, 4, 5, 6, 7);
}

// MFMA m of one half stage (every recipe but block-128): 8-bit operands
// issue 16 (tile i = m / 4, j = m % 4, one K=64 step), 16-bit operands 32
// (K=16 step s = m / 16 of the half, then i, j), E2M1 operands 32 (K=64
// step p = m / 16 of the half, then i, j).
//
// E2M1 on v_mfma_scale_f32_32x32x64_f8f6f4 (format 4): a lane's operand is
// its first four dwords, the 32 consecutive values K 32 lg .. 32 lg + 31 of
// the step (low nibble first), and the lane's E8M0 scale applies to exactly
// those 32 values (probed on gfx950).  One 16-byte LDS chunk is therefore one
// lane's whole operand and one MX block: step p of half h takes chunk
// 4 h + 2 p + lg, whose scale is byte 2 p + lg of the row's scale dword h.
// mxa / mxb then hold the words of dword h.
//
// MXFP8: the instruction's op_sel picks the scale byte, one choice for the
// whole wave, while the two lane groups need neighbouring bytes; the scale
// words are kept shifted right by 8 lg (once, as they are read from LDS), so
// byte 2 h of a lane's word is its own block's scale and no per-instruction
// byte extraction is needed (1-2% faster).  MXFP4 keeps the extraction: the
// same change made it 2-6% slower.
template <int OP, int SC, int AFMT, int BFMT>
__device__ __forceinline__ void mfma_one(f32x16 (&acc)[4][4], const Frags& f, const uint32_t* mxa,
                                         const uint32_t* mxb, int h, int lg, int m) {
  if (OP == OP_FP4) {
    const int p = m >> 4, i = (m >> 2) & 3, j = m & 3;
    const int sa_ = (int)((mxa[i] >> (8 * (2 * p + lg))) & 0xFFu);
    const int sb_ = (int)((mxb[j] >> (8 * (2 * p + lg))) & 0xFFu);
    const i32x4 a = f.a[i][p], b = f.b[j][p];
    const i32x8 a8 = __builtin_shufflevector(a, a, 0, 1, 2, 3, 0, 1, 2, 3);
    const i32x8 b8 = __builtin_shufflevector(b, b, 0, 1, 2, 3, 0, 1, 2, 3);
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[i][j], AFMT, BFMT, 0, sa_, 0, sb_);
  } else if (OP == OP_FP8) {
    const int i = m >> 2, j = m & 3;
    if (SC == SC_MX || SC == SC_MXC) {
      // the lane supplies the scale of MX block 2 h + lg of this stage
      if (h == 0)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cat(f.a[i]), cat(f.b[j]), acc[i][j], AFMT, BFMT,
                                                                     0, (int)mxa[i], 0, (int)mxb[j]);
      else
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cat(f.a[i]), cat(f.b[j]), acc[i][j], AFMT, BFMT,
                                                                     2, (int)mxa[i], 2, (int)mxb[j]);
    } else {
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cat(f.a[i]), cat(f.b[j]), acc[i][j], AFMT, BFMT,
                                                                   0, 0, 0, 0);
    }
  } else {
    const int s = m >> 4, i = (m >> 2) & 3, j = m & 3;
    const i32x4 a = f.a[i][s], b = f.b[j][s];
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                        acc[i][j], 0, 0, 0);
  }
}

// Share of n items that goes with MFMA m when n items are spread evenly over
// the first `over` MFMAs: items [n m / over, n (m + 1) / over).
__device__ __forceinline__ constexpr int share_lo(int n, int over, int m) { return m < over ? n * m / over : n; }
__device__ __forceinline__ constexpr int share_hi(int n, int over, int m) {
  return m < over ? n * (m + 1) / over : n;
}

// Epilogue shared by the kernels.  Lane (lr, lg) of tile (i, j) holds column
// 32 j + lr and rows 32 i + 8 (r / 4) + 4 lg + r % 4, r = 0..15.  Every LDS
// read of the main loop finished before its last barrier and no load is in
// flight, so the staging area may overwrite the tiles and the scale ring.
template <bool OUT_BF16>
__device__ __forceinline__ void store_tile(f32x16 (&acc)[4][4], const GemmArgs& g, uint8_t* smem, int m0, int n0,
                                           int w, int wm, int wn, int lane, float post) {
  const int lr = lane & 31, lg = lane >> 5;
  const bool full = (m0 + BM <= g.M) && (n0 + BN <= g.N);
  if constexpr (OUT_BF16) {
    // Lanes lr and lr ^ 1 swap half their values so that the even lane owns
    // rows R, R+1 and the odd lane rows R+2, R+3 of the column pair.
    const int par = lr & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float v0 = acc[i][j][4 * q] * post, v1 = acc[i][j][4 * q + 1] * post;
          const float v2 = acc[i][j][4 * q + 2] * post, v3 = acc[i][j][4 * q + 3] * post;
          const uint32_t own = par ? pk_bf16(v2, v3) : pk_bf16(v0, v1);
          const uint32_t snd = par ? pk_bf16(v0, v1) : pk_bf16(v2, v3);
          const uint32_t rcv = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)snd, 0xB1, 0xF, 0xF, false);
          const uint32_t lo = par ? rcv : own, hi = par ? own : rcv;
          const int row = wm * 128 + 32 * i + 8 * q + 4 * lg + 2 * par;
          const int colb = (wn * 128 + 32 * j + (lr & ~1)) * 2;
          *(uint32_t*)(smem + row * STG_BF16 + colb) = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
          *(uint32_t*)(smem + (row + 1) * STG_BF16 + colb) = __builtin_amdgcn_perm(hi, lo, 0x07060302u);
        }
    __syncthreads();
    const int ch = lane & 31;
    uint32_t mx = 0;
#pragma unroll 4
    for (int it = 0; it < 32; ++it) {
      const int s = 64 * w + 2 * it + (lane >> 5);
      const uint4 val = *(const uint4*)(smem + s * STG_BF16 + ch * 16);
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
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = wm * 64 + 32 * ii + 8 * (r >> 2) + 4 * lg + (r & 3);
            const int col = wn * 128 + 32 * j + lr;
            *(float*)(smem + row * STG_F32 + col * 4) = acc[2 * p + ii][j][r] * post;
          }
      __syncthreads();
#pragma unroll 4
      for (int it = 0; it < 32; ++it) {
        const int s = 32 * w + it;
        const uint4 val = *(const uint4*)(smem + s * STG_F32 + lane * 16);
        const int grow = m0 + (s >> 6) * 128 + 64 * p + (s & 63), gcol = n0 + lane * 4;
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

// ---------------------------------------------------------------------------
// The kernel.
//
// Schedule of K stage kt (LDS buffer b = kt & 1; f0 = fragments of its first
// half, already in registers):
//   phase A: MFMA(f0), interleaved with the reads f1 <- LDS b, second half
//   phase B: wait for this wave's loads, barrier: b^1 complete, nobody
//            reads b any more
//   phase C: MFMA(f1), interleaved with the loads of stage kt+2 into b and
//            the reads f0 <- LDS b^1, first half
// so LDS reads and global loads ride between MFMAs and global loads get
// about one stage of lead.  The last two stages are peeled (no loads, then
// no reads), so every phase is straight-line code.  Scale rows use a 3-deep
// LDS ring.  (Block-128 has its own kernel, gemm_blk.hip.)
//
// Epilogue: the accumulators go through LDS (bf16: adjacent lanes swap
// halves so each lane writes two 4-byte column pairs; fp32: 128 rows per
// pass), then every lane stores 16 contiguous bytes of C.
// ---------------------------------------------------------------------------
template <int OP, int LDA, int LDB, int SC, int AFMT, int BFMT, bool OUT_BF16>
__global__ __launch_bounds__(NTHR, 1) void gemm_kernel(GemmArgs g) {
  __shared__ __align__(16) uint8_t smem[smem_bytes(OP, SC)];
  constexpr bool MX = SC == SC_MX || SC == SC_MXC;

  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = w >> 1, wn = w & 1;
  int tm, tn;
  tile_of(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  constexpr int KST = (OP == OP_FP8) ? 128 : (OP == OP_FP4 ? 256 : 64);   // K elements per stage
  constexpr int SDW = sc_dw(OP);
  const int nk = g.K / KST;

  auto tileA = [&](int buf) { return smem + (buf * 2 + 0) * TILEB; };
  auto tileB = [&](int buf) { return smem + (buf * 2 + 1) * TILEB; };
  auto ring = [&](int slot, int o) { return (uint32_t*)(smem + SC_OFF + (slot * 2 + o) * BM * 4 * SDW); };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  Direct da, db;
  MnDirect ma, mb;
  RowDword sa, sb;
  if (LDA == LD_KMAJOR) direct_init(da, g.A, g.lda, m0, g.M, w);
  else mn_direct_init(ma, g.A, g.lda, m0, g.M, w);
  if (LDB == LD_KMAJOR) direct_init(db, g.B, g.ldb, n0, g.N, w);
  else mn_direct_init(mb, g.B, g.ldb, n0, g.N, w);
  if (MX) {
    rowdw_init(sa, g.a_scale, g.K / 32, m0, g.M, g.a_sdiv, w);
    rowdw_init(sb, g.b_scale, g.K / 32, n0, g.N, g.b_sdiv, w);
  }
  // SC_MXC: a lane loads 16 bytes of its row's scales at once (CH stages), one
  // load per row every CH stages instead of every stage.  Chunks are aligned
  // to the end of K: a chunk starts at stage s when s + delta is a multiple
  // of CH, delta = (CH - nk % CH) % CH; the first one may be shorter and its
  // 16-byte window then starts at stage 0.  Every window lies inside the row
  // (the host takes this path only when nk >= CH).  Chunk c sits in slot c % 2.
  constexpr int CH = 4 / SDW;
  const int delta = (CH - nk % CH) % CH;
  auto chunk_ws = [&](int s) {
    const int t0 = ((s + delta) / CH) * CH - delta;
    return t0 > 0 ? t0 : 0;
  };
  auto chunk_slot = [&](int s) { return ((s + delta) / CH) & 1; };
  auto chunk_start = [&](int s) { return s == 0 || (s + delta) % CH == 0; };
  auto ring16 = [&](int slot, int o) { return (uint32_t*)(smem + SC_OFF + (slot * 2 + o) * BM * 16); };
  auto chunk_issue = [&](int s) {
    const int ws = chunk_ws(s), slot = chunk_slot(s);
    __builtin_amdgcn_global_load_lds(sa.p + ws * SDW * 4, (lds_ptr_t)(ring16(slot, 0) + 64 * w * 4), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(sb.p + ws * SDW * 4, (lds_ptr_t)(ring16(slot, 1) + 64 * w * 4), 16, 0, 0);
  };

  auto issue = [&](int kt) {
    const int buf = kt & 1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (LDA == LD_KMAJOR) direct_item(da, kt, tileA(buf), w, i);
      else mn_direct_item(ma, kt, tileA(buf), w, i);
      if (LDB == LD_KMAJOR) direct_item(db, kt, tileB(buf), w, i);
      else mn_direct_item(mb, kt, tileB(buf), w, i);
    }
    if (SC == SC_MXC) {
      if (chunk_start(kt)) chunk_issue(kt);
    } else if (SC == SC_MX) {
      const int slot = kt % SC_RING;
      if (OP == OP_FP4) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          rowdw_issue_q<2>(sa, kt, q, ring(slot, 0), w);
          rowdw_issue_q<2>(sb, kt, q, ring(slot, 1), w);
        }
      } else {
        rowdw_issue(sa, kt, ring(slot, 0), w);
        rowdw_issue(sb, kt, ring(slot, 1), w);
      }
    }
  };
  const int lr = lane & 31, lg = lane >> 5;     // row within a 32-tile, K group
  const uint32_t lb = (uint32_t)(lr * 128 + ((lg ^ swz_key(lr)) << 4));
  // per-lane part of the MN-major transposing reads (see op_read)
  const int jj = (lr & 15) >> 2;
  const uint32_t lbm = (uint32_t)((8 * lg + jj) * 512 + 64 * jj + 32 * (lr >> 4) + 16 * ((lr & 3) >> 1) + 8 * (lr & 1));
  const uint32_t lba = LDA == LD_KMAJOR ? lb : lbm + 256 * wm;
  const uint32_t lbb = LDB == LD_KMAJOR ? lb : lbm + 256 * wn;
  // where the wave's fragments start within a tile: K-major tiles hold its
  // 128 rows at 128 x 128 B; MN-major tiles put its columns in lba / lbb
  const int offA = LDA == LD_KMAJOR ? wm * 16384 : 0, offB = LDB == LD_KMAJOR ? wn * 16384 : 0;

  constexpr int NMFMA = (OP == OP_FP8) ? 16 : 32;                // per half stage
  constexpr int VM_A = 8;
  constexpr int VM_B = 8;
  constexpr int VM_STAGE = VM_A + VM_B + (SC == SC_MX ? 2 * SDW : 0);
  constexpr int DS_HALF = op_reads<LDA>() + op_reads<LDB>();       // fragment reads per half stage
  constexpr int DS_NEXT = DS_HALF + (MX ? 8 : 0);
  // MXFP4: phase A also reads the stage's second scale dword (used in phase C)
  constexpr int DS_A = DS_HALF + (OP == OP_FP4 ? 8 : 0);
  Frags f0, f1;
  // MX scale words of the tiles: MXFP8 one dword per row and stage (mxa /
  // mxb, the next stage's in nxa / nxb); MXFP4 dword 0 in mxa / mxb (phase
  // A, refilled for the next stage in phase C) and dword 1 in m1a / m1b
  // (read in phase A, used in phase C)
  uint32_t mxa[4] = {0, 0, 0, 0}, mxb[4] = {0, 0, 0, 0};
  uint32_t m1a[4] = {0, 0, 0, 0}, m1b[4] = {0, 0, 0, 0};
  constexpr int HALF = NMFMA / 2;

  // global load v (of VM_STAGE) of stage kt
  auto issue_item = [&](int kt, int v) {
    const int buf = kt & 1;
    if (v < VM_A) {
      if (LDA == LD_KMAJOR) direct_item(da, kt, tileA(buf), w, v);
      else mn_direct_item(ma, kt, tileA(buf), w, v);
    } else if (v < VM_A + VM_B) {
      const int u = v - VM_A;
      if (LDB == LD_KMAJOR) direct_item(db, kt, tileB(buf), w, u);
      else mn_direct_item(mb, kt, tileB(buf), w, u);
    } else {
      const int slot = kt % SC_RING;
      const int u = v - VM_A - VM_B;
      if (OP == OP_FP4) rowdw_issue_q<2>((u & 1) ? sb : sa, kt, u >> 1, ring(slot, u & 1), w);
      else if (u == 0) rowdw_issue(sa, kt, ring(slot, 0), w);
      else rowdw_issue(sb, kt, ring(slot, 1), w);
    }
  };
  // LDS read e (of 8) of the MX scale words (dword q) of stage kt; MXFP8's
  // are shifted right by 8 lg for the MFMA's byte select (see mfma_one)
  const uint32_t mxsh = OP == OP_FP4 ? 0u : 8u * (uint32_t)lg;
  auto mx_item = [&](uint32_t* xa, uint32_t* xb, int kt, int e, int q) {
    if (SC == SC_MXC) {
      const int slot = chunk_slot(kt), wd = (kt - chunk_ws(kt)) * SDW + q;
      if (e < 4) xa[e] = ring16(slot, 0)[(wm * 128 + 32 * e + lr) * 4 + wd] >> mxsh;
      else xb[e - 4] = ring16(slot, 1)[(wn * 128 + 32 * (e - 4) + lr) * 4 + wd] >> mxsh;
    } else {
      const int slot = kt % SC_RING;
      if (e < 4) xa[e] = ring(slot, 0)[q * BM + wm * 128 + 32 * e + lr] >> mxsh;
      else xb[e - 4] = ring(slot, 1)[q * BM + wn * 128 + 32 * (e - 4) + lr] >> mxsh;
    }
  };

  issue(0);
  wait_vm0();
  __syncthreads();
  if (nk > 1) issue(1);
#pragma unroll
  for (int d = 0; d < DS_HALF; ++d) frag_read<0, LDA, LDB>(f0, d, tileA(0) + offA, tileB(0) + offB, lba, lbb);
  if (MX) {
#pragma unroll
    for (int e = 0; e < 8; ++e) mx_item(mxa, mxb, 0, e, 0);
  }

  auto body = [&](int kt, auto issue_c, auto next_c) {
    constexpr bool ISSUE = decltype(issue_c)::value;
    constexpr bool NEXT = decltype(next_c)::value;
    const int buf = kt & 1;
    const uint8_t* curA = tileA(buf) + offA;
    const uint8_t* curB = tileB(buf) + offB;
    const uint8_t* nxtA = tileA(buf ^ 1) + offA;
    const uint8_t* nxtB = tileB(buf ^ 1) + offB;
    // phase A: MFMA(f0); the reads of f1 ride on the first half of the MFMAs
#pragma unroll
    for (int m = 0; m < NMFMA; ++m) {
      mfma_one<OP, SC, AFMT, BFMT>(acc, f0, mxa, mxb, 0, lg, m);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int d = share_lo(DS_A, HALF, m); d < share_hi(DS_A, HALF, m); ++d) {
        if (d < DS_HALF) frag_read<1, LDA, LDB>(f1, d, curA, curB, lba, lbb);
        else mx_item(m1a, m1b, kt, d - DS_HALF, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // phase B: this wave's loads of stage kt+1 (tiles and scale words) have
    // landed, then every wave's.  The wait is explicit: the compiler adds
    // one only where it cannot tell an LDS read from the loads in flight,
    // which depends on how it scheduled the reads.
    wait_vm0();
    __syncthreads();
    // SC_MXC: the scale chunk that starts at stage kt+2 goes with its tiles
    if (SC == SC_MXC && ISSUE) {
      if (chunk_start(kt + 2)) chunk_issue(kt + 2);
    }
    __builtin_amdgcn_sched_barrier(0);
    // phase C: MFMA(f1); reads of the next f0 (and MX words) on the first
    // half of the MFMAs, the loads of stage kt+2 spread over all of them
    uint32_t nxa[4] = {0, 0, 0, 0}, nxb[4] = {0, 0, 0, 0};
    constexpr int NDS = NEXT ? DS_NEXT : 0;
    constexpr int NVM = ISSUE ? VM_STAGE : 0;
#pragma unroll
    for (int m = 0; m < NMFMA; ++m) {
      if (OP == OP_FP4) mfma_one<OP, SC, AFMT, BFMT>(acc, f1, m1a, m1b, 1, lg, m);
      else mfma_one<OP, SC, AFMT, BFMT>(acc, f1, mxa, mxb, 1, lg, m);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int d = share_lo(NDS, HALF, m); d < share_hi(NDS, HALF, m); ++d) {
        if (d < DS_HALF) frag_read<0, LDA, LDB>(f0, d, nxtA, nxtB, lba, lbb);
        else if (OP == OP_FP4) mx_item(mxa, mxb, kt + 1, d - DS_HALF, 0);
        else mx_item(nxa, nxb, kt + 1, d - DS_HALF, 0);
      }
#pragma unroll
      for (int v = share_lo(NVM, NMFMA, m); v < share_hi(NVM, NMFMA, m); ++v) issue_item(kt + 2, v);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (NEXT && MX && OP != OP_FP4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        mxa[i] = nxa[i];
        mxb[i] = nxb[i];
      }
    }
  };
  using T_ = std::integral_constant<bool, true>;
  using F_ = std::integral_constant<bool, false>;
  for (int kt = 0; kt < nk - 2; ++kt) body(kt, T_{}, T_{});
  if (nk >= 2) body(nk - 2, F_{}, T_{});
  body(nk - 1, F_{}, F_{});

  float post = 1.0f;
  if (SC == SC_TENSOR) post = (*g.a_ts) * (*g.b_ts);
  if constexpr (SC == SC_CHAN) {
    // acc[i][j][4 q + r] is C[row, col] with row = m0 + 128 wm + 32 i + 8 q +
    // 4 lg + r, col = n0 + 128 wn + 32 j + lr (store_tile's lane layout);
    // rows and columns past the end read the last scale (never stored)
    const float* sa = (const float*)g.a_scale;
    const float* sb = (const float*)g.b_scale;
    const int lr = lane & 31, lg = lane >> 5;
    float fb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + 128 * wn + 32 * j + lr;
      fb[j] = sb[n < g.N ? n : g.N - 1];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int mr = m0 + 128 * wm + 32 * i + 8 * q + 4 * lg;   // a multiple of 4, as is M
        const float4 s4 = *(const float4*)(sa + (mr < g.M ? mr : g.M - 4));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j][4 * q + 0] *= s4.x * fb[j];
          acc[i][j][4 * q + 1] *= s4.y * fb[j];
          acc[i][j][4 * q + 2] *= s4.z * fb[j];
          acc[i][j][4 * q + 3] *= s4.w * fb[j];
        }
      }
  }
  store_tile<OUT_BF16>(acc, g, smem, m0, n0, w, wm, wn, lane, post);
}

// ---------------------------------------------------------------------------
// NVFP4 kernel: raw E2M1 tiles in LDS, decoded per fragment.
//
// A K stage is 128 values = 64 bytes of every operand row, loaded straight
// into LDS (global_load_lds_dwordx4), with the stage's 8 block-scale bytes
// per row next to it.  Row r's 16-byte chunk c sits at r * 64 + ((c ^ key)
// << 4), key = (r >> 2) & 3, which makes the 16-lane fragment reads
// conflict-free.
//
// Lane (lr, lg) of a 32-row tile reads chunk 2 h + lg of its row for half
// stage h: 32 values, of which dword d (values 8 d .. 8 d + 7 of the chunk)
// is its operand of K=16 step d of the half.  The contraction index of the
// stage is thereby permuted (step d of half h takes values 64 h + 8 d + {0..7}
// from lane group 0 and 64 h + 32 + 8 d + {0..7} from lane group 1), the same
// way for A and B, which leaves every sum over K unchanged.  Each operand
// dword decodes exactly into 8 fp16: v_cvt_scalef32_pk_f16_fp4 (scale 1)
// and a multiply by the E4M3 block scale converted to fp16 (the product has
// at most 6 significant bits and lies in [2^-10, 2688]).  Values 8 d .. 8 d +
// 7 of chunk 2 h + lg belong to block 4 h + 2 lg + d / 2 of the stage.
//
// Per half stage a wave runs 4 steps x 16 MFMAs (32x32x16 f16) and decodes
// the next step's 8 operands (4 A and 4 B tiles) between them; the LDS reads
// of the next half's raw chunks and the next stage's global loads ride on the
// same MFMAs.  Phases A / B / C and the peeled tail are as in gemm_kernel.
// ---------------------------------------------------------------------------
constexpr int NV_ROWB = 64;                   // bytes per row per stage (K = 128)
constexpr int NV_TILE = BM * NV_ROWB;         // 16 KB per operand per stage
constexpr int NV_SC = BM * 8;                 // 8 scale bytes per row per stage
constexpr int NV_SC_OFF = 4 * NV_TILE;

__device__ __forceinline__ int nv_key(int row) { return (row >> 2) & 3; }

struct NvDirect {
  const uint8_t* base;
  uint32_t off[4];
};

// load i (of 4) of wave w fills rows 16 q .. 16 q + 15, q = 4 w + i; lane l
// owns row 16 q + l / 4, physical chunk l % 4.
__device__ __forceinline__ void nv_direct_init(NvDirect& d, const uint8_t* p, int64_t ld, int rows0, int nrows,
                                               int w) {
  const int lane = threadIdx.x & 63;
  d.base = p + (int64_t)rows0 * ld;
  const int lim = nrows - rows0 - 1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int trow = 16 * (4 * w + i) + (lane >> 2);
    const int lc = (lane & 3) ^ nv_key(trow);
    const int r = trow < lim ? trow : lim;
    d.off[i] = (uint32_t)r * (uint32_t)ld + (uint32_t)(lc << 4);
  }
}

// (global_load_lds: the buffer-resource form that Direct uses measured 0.6%
// slower here, the compiler then splitting the raw-chunk waits)
__device__ __forceinline__ void nv_direct_item(const NvDirect& d, int kt, uint8_t* tile, int w, int i) {
  __builtin_amdgcn_global_load_lds(d.base + (int64_t)kt * NV_ROWB + d.off[i],
                                   (lds_ptr_t)(tile + (4 * w + i) * 1024), 16, 0, 0);
}

// Scale rows: load i (of 2) of wave w fills rows 32 q .. 32 q + 31, q = 2 w + i,
// one dword per lane (lane l: row 32 q + l / 2, dword l % 2).
struct NvScale {
  const uint8_t* p[2];
};

__device__ __forceinline__ void nv_scale_init(NvScale& s, const uint8_t* scale, int K, int rows0, int nrows,
                                              bool twod, int w) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    int row = rows0 + 32 * (2 * w + i) + (lane >> 1);
    row = row < nrows ? row : nrows - 1;
    const int64_t srow = twod ? row / 16 : row;
    s.p[i] = scale + srow * (int64_t)(K / 16) + (lane & 1) * 4;
  }
}

__device__ __forceinline__ void nv_scale_item(const NvScale& s, int kt, uint8_t* ring_slot, int w, int i) {
  __builtin_amdgcn_global_load_lds(s.p[i] + (int64_t)kt * 8, (lds_ptr_t)(ring_slot + (2 * w + i) * 256), 4, 0, 0);
}

// 8 E2M1 codes (element 2k in the low nibble of byte k) times an fp16 scale,
// as the fp16 operand of one K=16 step.
__device__ __forceinline__ i32x4 nv_decode(uint32_t raw, f16x2 sc) {
  // the four conversions first, then the four multiplies: each multiply
  // waits for its conversion's result, and four independent chains hide
  // that latency where one register reused for every pair would not
  const f16x2 c0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(raw, 1.0f, 0);
  const f16x2 c1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(raw, 1.0f, 1);
  const f16x2 c2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(raw, 1.0f, 2);
  const f16x2 c3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(raw, 1.0f, 3);
  const f16x2 p0 = c0 * sc, p1 = c1 * sc, p2 = c2 * sc, p3 = c3 * sc;
  i32x4 r;
  r.x = __builtin_bit_cast(int, p0);
  r.y = __builtin_bit_cast(int, p1);
  r.z = __builtin_bit_cast(int, p2);
  r.w = __builtin_bit_cast(int, p3);
  return r;
}

// The two E4M3 block scales of one lane for one half stage (blocks
// 4 h + 2 lg and + 1), exactly as fp16 (v_cvt_scalef32_pk_f16_fp8, scale 1).
__device__ __forceinline__ f16x2 nv_scale_pair(uint32_t dword_h, int sh) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(dword_h >> sh, 1.0f, false);
}

template <bool B2D, bool OUT_BF16>
__global__ __launch_bounds__(NTHR, 1) void gemm_nvfp4_kernel(GemmArgs g) {
  __shared__ __align__(16) uint8_t smem[SMEM];

  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = w >> 1, wn = w & 1;
  int tm, tn;
  tile_of(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int nk = g.K / 128;

  auto tileA = [&](int buf) { return smem + (buf * 2 + 0) * NV_TILE; };
  auto tileB = [&](int buf) { return smem + (buf * 2 + 1) * NV_TILE; };
  auto ring = [&](int slot, int o) { return smem + NV_SC_OFF + (slot * 2 + o) * NV_SC; };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  NvDirect da, db;
  NvScale sa, sb;
  nv_direct_init(da, g.A, g.lda, m0, g.M, w);
  nv_direct_init(db, g.B, g.ldb, n0, g.N, w);
  nv_scale_init(sa, g.a_scale, g.K, m0, g.M, false, w);
  nv_scale_init(sb, g.b_scale, g.K, n0, g.N, B2D, w);

  constexpr int NVM = 12;              // global loads per stage and wave: 4 + 4 data, 2 + 2 scales
  auto issue_item = [&](int kt, int v) {
    const int buf = kt & 1, slot = kt % SC_RING;
    if (v < 4) nv_direct_item(da, kt, tileA(buf), w, v);
    else if (v < 8) nv_direct_item(db, kt, tileB(buf), w, v - 4);
    else if (v < 10) nv_scale_item(sa, kt, ring(slot, 0), w, v - 8);
    else nv_scale_item(sb, kt, ring(slot, 1), w, v - 10);
  };

  const int lr = lane & 31, lg = lane >> 5;
  const int key = nv_key(lr);
  const uint32_t lb[2] = {(uint32_t)(lr * NV_ROWB + (((0 + lg) ^ key) << 4)),
                          (uint32_t)(lr * NV_ROWB + (((2 + lg) ^ key) << 4))};
  const int sh = 16 * lg;
  const int rowA = wm * 128, rowB = wn * 128;

  // raw[0] / raw[1]: halves 0 / 1 of the stage being multiplied; raw[2]:
  // half 1 of the next stage (read in phase C while raw[1] is still in use)
  uint4 raw[3][8];          // [buffer][tile: 0-3 A, 4-7 B]
  uint2 scw[8], scn[8];     // this stage's / the next stage's scale bytes per tile row
  i32x4 dec[2][8];          // decoded operands of two consecutive K=16 steps
  f16x2 sp[8];              // fp16 block-scale pair of the half being decoded

  // raw read e (of 8) of half h from the tiles at pa / pb (this wave's rows);
  // scale read e (of 8) from the ring slot rows at qa / qb
  auto raw_item = [&](uint4* dst, const uint8_t* pa, const uint8_t* pb, int h, int e) {
    const uint8_t* base = (e < 4) ? pa + (32 * e) * NV_ROWB : pb + (32 * (e - 4)) * NV_ROWB;
    dst[e] = *(const uint4*)(base + lb[h]);
  };
  auto sc_item = [&](uint2* dst, const uint8_t* qa, const uint8_t* qb, int e) {
    const uint8_t* base = (e < 4) ? qa + (32 * e) * 8 : qb + (32 * (e - 4)) * 8;
    dst[e] = *(const uint2*)base;
  };
  auto set_scales = [&](const uint2* s, int h) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sp[e] = nv_scale_pair(h ? s[e].y : s[e].x, sh);
  };
  // decode operand e (of 8) of step d of the half held in raw[r] into dec[slot]
  auto dec_item = [&](int slot, int r, int d, int e) {
    const uint32_t rw = d == 0 ? raw[r][e].x : d == 1 ? raw[r][e].y : d == 2 ? raw[r][e].z : raw[r][e].w;
    const f16x2 s2 = d < 2 ? __builtin_shufflevector(sp[e], sp[e], 0, 0) : __builtin_shufflevector(sp[e], sp[e], 1, 1);
    dec[slot][e] = nv_decode(rw, s2);
  };
  auto mfma_item = [&](int slot, int m) {
    const int i = m >> 2, j = m & 3;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, dec[slot][i]),
                                                       __builtin_bit_cast(f16x8, dec[slot][4 + j]), acc[i][j], 0, 0, 0);
  };

  // prologue: stage 0 in LDS, stage 1 in flight, stage 0 read, step 0 decoded
#pragma unroll
  for (int v = 0; v < NVM; ++v) issue_item(0, v);
  wait_vm0();
  __syncthreads();
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    raw_item(raw[0], tileA(0) + rowA * NV_ROWB, tileB(0) + rowB * NV_ROWB, 0, e);
    raw_item(raw[1], tileA(0) + rowA * NV_ROWB, tileB(0) + rowB * NV_ROWB, 1, e);
    sc_item(scw, ring(0, 0) + (rowA + lr) * 8, ring(0, 1) + (rowB + lr) * 8, e);
  }
  if (nk > 1) {
#pragma unroll
    for (int v = 0; v < NVM; ++v) issue_item(1, v);
  }
  set_scales(scw, 0);
#pragma unroll
  for (int e = 0; e < 8; ++e) dec_item(0, 0, 0, e);

  // One stage: 8 steps of 16 MFMAs on dec[d & 1]; between them the decode of
  // the following step (one operand per 2 MFMAs).  All LDS reads of a stage
  // (the next stage's raw chunks and scales) come first in phase C and all
  // its global loads after them, so no LDS read ever waits behind a load
  // that is still writing LDS.
  auto body = [&](int kt, auto issue_c, auto next_c) {
    constexpr bool ISSUE = decltype(issue_c)::value;
    constexpr bool NEXT = decltype(next_c)::value;
    const int buf = kt & 1, nslot = (kt + 1) % SC_RING;
    const uint8_t* nxtA = tileA(buf ^ 1) + rowA * NV_ROWB;
    const uint8_t* nxtB = tileB(buf ^ 1) + rowB * NV_ROWB;
    const uint8_t* nqa = ring(nslot, 0) + (rowA + lr) * 8;
    const uint8_t* nqb = ring(nslot, 1) + (rowB + lr) * 8;
    // phase A: half 0 (raw[0]); its last step decodes half 1's first
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      if (d == 3) set_scales(scw, 1);
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        mfma_item(d & 1, m);
        __builtin_amdgcn_sched_barrier(0);
        if ((m & 1) == 1) {
          if (d < 3) dec_item((d + 1) & 1, 0, d + 1, m >> 1);
          else dec_item(0, 1, 0, m >> 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // phase B: this wave's loads of stage kt+1 have landed (explicit wait,
    // as in gemm_kernel), then every wave's
    wait_vm0();
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    // phase C: half 1 (raw[1]); steps 0-1 read the next stage (24 LDS
    // reads), steps 2-3 issue the loads of stage kt+2 (12)
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      if (d == 3 && NEXT) set_scales(scn, 0);
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        mfma_item(d & 1, m);
        __builtin_amdgcn_sched_barrier(0);
        if (NEXT && d == 0 && m < 8) raw_item(raw[0], nxtA, nxtB, 0, m);
        if (NEXT && d == 0 && m >= 8) raw_item(raw[2], nxtA, nxtB, 1, m - 8);
        if (NEXT && d == 1 && m < 8) sc_item(scn, nqa, nqb, m);
        if (ISSUE && d >= 2 && m < 12 && (m & 1) == 0) issue_item(kt + 2, (d - 2) * 6 + (m >> 1));
        if ((m & 1) == 1) {
          if (d < 3) dec_item((d + 1) & 1, 1, d + 1, m >> 1);
          else if (NEXT) dec_item(0, 0, 0, m >> 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (NEXT) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        scw[e] = scn[e];
        raw[1][e] = raw[2][e];
      }
    }
  };
  using T_ = std::integral_constant<bool, true>;
  using F_ = std::integral_constant<bool, false>;
  for (int kt = 0; kt < nk - 2; ++kt) body(kt, T_{}, T_{});
  if (nk >= 2) body(nk - 2, F_{}, T_{});
  body(nk - 1, F_{}, F_{});

  store_tile<OUT_BF16>(acc, g, smem, m0, n0, w, wm, wn, lane, (*g.a_ts) * (*g.b_ts));
}

__global__ void zero_c_kernel(uint8_t* c, int64_t bytes) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < bytes; i += (int64_t)gridDim.x * blockDim.x)
    c[i] = 0;
}


template <int OP, int LDA, int LDB, int SC, int AFMT, int BFMT>
static gemm_fn pick_out(bool bf16_out) {
  return bf16_out ? gemm_kernel<OP, LDA, LDB, SC, AFMT, BFMT, true> : gemm_kernel<OP, LDA, LDB, SC, AFMT, BFMT, false>;
}

template <int SC>
static gemm_fn pick_fp8(int afmt, int bfmt, bool bf16_out) {
  if (afmt == 0 && bfmt == 0) return pick_out<OP_FP8, LD_KMAJOR, LD_KMAJOR, SC, 0, 0>(bf16_out);
  if (afmt == 1 && bfmt == 0) return pick_out<OP_FP8, LD_KMAJOR, LD_KMAJOR, SC, 1, 0>(bf16_out);
  if (afmt == 0 && bfmt == 1) return pick_out<OP_FP8, LD_KMAJOR, LD_KMAJOR, SC, 0, 1>(bf16_out);
  return pick_out<OP_FP8, LD_KMAJOR, LD_KMAJOR, SC, 1, 1>(bf16_out);
}

}  // namespace pbs

using namespace pbs;

__global__ void zero_word_kernel(uint32_t* p) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *p = 0u;
}

// pbs_gemm, and with c_amax non-null pbs_gemm_amax: the epilogue also folds
// max |C| of the stored values into *c_amax (reset to 0 first, stream-ordered).
static pbs_status gemm_impl(pbs_recipe recipe, pbs_layout layout, int64_t M, int64_t N, int64_t K,
                            const void* A, pbs_format a_fmt, const void* a_scale,
                            const float* a_tensor_scale, const void* B, pbs_format b_fmt,
                            const void* b_scale, const float* b_tensor_scale, void* C,
                            pbs_format c_fmt, float* c_amax, hipStream_t stream) {
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
  if (M == 0 || N == 0) {
    if (!c_amax) return PBS_OK;
    hipLaunchKernelGGL(zero_word_kernel, dim3(1), dim3(64), 0, stream, (uint32_t*)c_amax);
    return check_launch("pbs_gemm");
  }
  if (K == 0) {
    if (c_amax) hipLaunchKernelGGL(zero_word_kernel, dim3(1), dim3(64), 0, stream, (uint32_t*)c_amax);
    const int64_t bytes = M * N * (bf16_out ? 2 : 4);
    hipLaunchKernelGGL(zero_c_kernel, dim3(1024), dim3(256), 0, stream, (uint8_t*)C, bytes);
    return check_launch("pbs_gemm");
  }
  PBS_REQUIRE(A && B, PBS_ERR_INVALID_ARG, "pbs_gemm: A or B is null");
  PBS_REQUIRE(((uintptr_t)A & 15) == 0 && ((uintptr_t)B & 15) == 0, PBS_ERR_INVALID_ARG,
              "pbs_gemm: A and B must be 16-byte aligned");
  PBS_REQUIRE(((uintptr_t)C & 15) == 0, PBS_ERR_INVALID_ARG, "pbs_gemm: C must be 16-byte aligned");

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
  g.tiles_m = (int)ceil_div(M, BM);
  g.tiles_n = (int)ceil_div(N, BN);
  g.a_sdiv = 1;
  g.b_sdiv = 1;
  g.c_amax = (uint32_t*)c_amax;

  gemm_fn fn = nullptr;
  int nthr = NTHR;                     // threads per workgroup of the chosen kernel
  const char* name = "";
  const bool w2d = layout != PBS_WGRAD;     // weights carry 2D block scales
  switch (recipe) {
    case PBS_RECIPE_BF16: {
      PBS_REQUIRE(a_fmt == PBS_FMT_BF16 && b_fmt == PBS_FMT_BF16, PBS_ERR_UNSUPPORTED,
                  "pbs_gemm: BF16 recipe takes BF16 operands");
      PBS_REQUIRE(K % 64 == 0, PBS_ERR_SHAPE, "pbs_gemm: BF16 needs K %% 64 == 0");
      if (layout == PBS_FPROP) {
        g.lda = K * 2; g.ldb = K * 2;
        fn = pick_out<OP_BF16, LD_KMAJOR, LD_KMAJOR, SC_NONE, 0, 0>(bf16_out);
      } else if (layout == PBS_DGRAD) {
        g.lda = K * 2; g.ldb = N * 2;               // B = W stored [K, N]
        fn = pick_out<OP_BF16, LD_KMAJOR, LD_MNMAJOR, SC_NONE, 0, 0>(bf16_out);
      } else {
        g.lda = M * 2; g.ldb = N * 2;               // A = X stored [K, M], B = dY stored [K, N]
        fn = pick_out<OP_BF16, LD_MNMAJOR, LD_MNMAJOR, SC_NONE, 0, 0>(bf16_out);
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
      fn = pick_fp8<SC_TENSOR>(a_fmt == PBS_FMT_E5M2, b_fmt == PBS_FMT_E5M2, bf16_out);
      name = "gemm_fp8_tensor";
      break;
    }
    case PBS_RECIPE_FP8_CHANNEL: {
      PBS_REQUIRE(a_fmt == PBS_FMT_E4M3 && b_fmt == PBS_FMT_E4M3, PBS_ERR_UNSUPPORTED,
                  "pbs_gemm: FP8_CHANNEL takes E4M3 operands");
      PBS_REQUIRE(a_scale && b_scale, PBS_ERR_INVALID_ARG, "pbs_gemm: channel scales are null");
      PBS_REQUIRE(((uintptr_t)a_scale & 15) == 0 && ((uintptr_t)b_scale & 15) == 0, PBS_ERR_INVALID_ARG,
                  "pbs_gemm: FP8_CHANNEL scales must be 16-byte aligned");
      PBS_REQUIRE(K % 128 == 0, PBS_ERR_SHAPE, "pbs_gemm: FP8 needs K %% 128 == 0");
      g.lda = K; g.ldb = K;
      fn = pick_out<OP_FP8, LD_KMAJOR, LD_KMAJOR, SC_CHAN, 0, 0>(bf16_out);
      name = "gemm_fp8_channel";
      break;
    }
    case PBS_RECIPE_FP8_BLOCK128: {
      PBS_REQUIRE(a_fmt == PBS_FMT_E4M3 && b_fmt == PBS_FMT_E4M3, PBS_ERR_UNSUPPORTED,
                  "pbs_gemm: FP8_BLOCK128 takes E4M3 operands");
      PBS_REQUIRE(a_scale && b_scale, PBS_ERR_INVALID_ARG, "pbs_gemm: block scales are null");
      PBS_REQUIRE(K % 128 == 0, PBS_ERR_SHAPE, "pbs_gemm: FP8_BLOCK128 needs K %% 128 == 0");
      PBS_REQUIRE(!w2d || N % 128 == 0, PBS_ERR_SHAPE, "pbs_gemm: 128x128 weight blocks need N %% 128 == 0");
      g.lda = K; g.ldb = K;
      g.tiles_n = (int)ceil_div(N, BLK_BN);       // gemm_blk.hip: 256 x 256 tiles, 8 waves
      nthr = BLK_THR;
      fn = blk_kernel_for(false, w2d, bf16_out);
      name = "gemm_fp8_block128";
      break;
    }
    case PBS_RECIPE_FP8_BLOCK128_1D1D:
    case PBS_RECIPE_FP8_BLOCK128_2D2D: {
      const bool two = recipe == PBS_RECIPE_FP8_BLOCK128_2D2D;
      PBS_REQUIRE(a_fmt == PBS_FMT_E4M3 && b_fmt == PBS_FMT_E4M3, PBS_ERR_UNSUPPORTED,
                  "pbs_gemm: sub-channel FP8 takes E4M3 operands");
      PBS_REQUIRE(a_scale && b_scale, PBS_ERR_INVALID_ARG, "pbs_gemm: block scales are null");
      PBS_REQUIRE(K % 128 == 0, PBS_ERR_SHAPE, "pbs_gemm: sub-channel FP8 needs K %% 128 == 0");
      PBS_REQUIRE(!two || (M % 128 == 0 && N % 128 == 0), PBS_ERR_SHAPE,
                  "pbs_gemm: 128x128 blocks on both operands need M and N %% 128 == 0");
      g.lda = K; g.ldb = K;
      g.tiles_n = (int)ceil_div(N, BLK_BN);
      nthr = BLK_THR;
      fn = blk_kernel_for(two, two, bf16_out);
      name = two ? "gemm_fp8_block128_2d2d" : "gemm_fp8_block128_1d1d";
      break;
    }
    case PBS_RECIPE_MXFP8: {
      PBS_REQUIRE(a_fmt == PBS_FMT_E4M3 && b_fmt == PBS_FMT_E4M3, PBS_ERR_UNSUPPORTED,
                  "pbs_gemm: MXFP8 takes E4M3 operands");
      PBS_REQUIRE(a_scale && b_scale, PBS_ERR_INVALID_ARG, "pbs_gemm: block scales are null");
      PBS_REQUIRE(K % 128 == 0, PBS_ERR_SHAPE, "pbs_gemm: MXFP8 needs K %% 128 == 0");
      PBS_REQUIRE(((uintptr_t)a_scale & 3) == 0 && ((uintptr_t)b_scale & 3) == 0, PBS_ERR_INVALID_ARG,
                  "pbs_gemm: MXFP8 block scales must be 4-byte aligned");
      g.lda = K; g.ldb = K;
      // scale rows in 16-byte chunks once the row holds 4 stages of them
      fn = K / 128 >= 4 ? pick_out<OP_FP8, LD_KMAJOR, LD_KMAJOR, SC_MXC, 0, 0>(bf16_out)
                        : pick_out<OP_FP8, LD_KMAJOR, LD_KMAJOR, SC_MX, 0, 0>(bf16_out);
      name = "gemm_mxfp8";
      break;
    }
    case PBS_RECIPE_FP8_BLOCK128_POW2: {
      // Power-of-two block scales ride on the scaled MFMA like MXFP8's: each
      // 128-long K stage is one block, whose scale word holds its E8M0 code
      // in all four bytes, so every 32-value step of the stage reads it.
      PBS_REQUIRE(a_fmt == PBS_FMT_E4M3 && b_fmt == PBS_FMT_E4M3, PBS_ERR_UNSUPPORTED,
                  "pbs_gemm: FP8_BLOCK128_POW2 takes E4M3 operands");
      PBS_REQUIRE(a_scale && b_scale, PBS_ERR_INVALID_ARG, "pbs_gemm: block scales are null");
      PBS_REQUIRE(K % 128 == 0, PBS_ERR_SHAPE, "pbs_gemm: FP8_BLOCK128_POW2 needs K %% 128 == 0");
      PBS_REQUIRE(!w2d || N % 128 == 0, PBS_ERR_SHAPE, "pbs_gemm: 128x128 weight blocks need N %% 128 == 0");
      PBS_REQUIRE(((uintptr_t)a_scale & 3) == 0 && ((uintptr_t)b_scale & 3) == 0, PBS_ERR_INVALID_ARG,
                  "pbs_gemm: FP8_BLOCK128_POW2 scale words must be 4-byte aligned");
      g.lda = K; g.ldb = K;
      g.b_sdiv = w2d ? 128 : 1;                   // 128x128 weight blocks: one scale row per 128 rows
      fn = K / 128 >= 4 ? pick_out<OP_FP8, LD_KMAJOR, LD_KMAJOR, SC_MXC, 0, 0>(bf16_out)
                        : pick_out<OP_FP8, LD_KMAJOR, LD_KMAJOR, SC_MX, 0, 0>(bf16_out);
      name = "gemm_fp8_block128_pow2";
      break;
    }
    case PBS_RECIPE_MXFP4: {
      PBS_REQUIRE(a_fmt == PBS_FMT_E2M1 && b_fmt == PBS_FMT_E2M1, PBS_ERR_UNSUPPORTED,
                  "pbs_gemm: MXFP4 takes E2M1 operands");
      PBS_REQUIRE(a_scale && b_scale, PBS_ERR_INVALID_ARG, "pbs_gemm: block scales are null");
      PBS_REQUIRE(K % 256 == 0, PBS_ERR_SHAPE, "pbs_gemm: MXFP4 needs K %% 256 == 0");
      PBS_REQUIRE(((uintptr_t)a_scale & 3) == 0 && ((uintptr_t)b_scale & 3) == 0, PBS_ERR_INVALID_ARG,
                  "pbs_gemm: MXFP4 block scales must be 4-byte aligned");
      g.lda = K / 2; g.ldb = K / 2;
      fn = K / 256 >= 2 ? pick_out<OP_FP4, LD_KMAJOR, LD_KMAJOR, SC_MXC, 4, 4>(bf16_out)
                        : pick_out<OP_FP4, LD_KMAJOR, LD_KMAJOR, SC_MX, 4, 4>(bf16_out);
      name = "gemm_mxfp4";
      break;
    }
    case PBS_RECIPE_NVFP4: {
      PBS_REQUIRE(a_fmt == PBS_FMT_E2M1 && b_fmt == PBS_FMT_E2M1, PBS_ERR_UNSUPPORTED,
                  "pbs_gemm: NVFP4 takes E2M1 operands");
      PBS_REQUIRE(a_scale && b_scale && a_tensor_scale && b_tensor_scale, PBS_ERR_INVALID_ARG,
                  "pbs_gemm: NVFP4 needs block and tensor scales");
      PBS_REQUIRE(K % 128 == 0, PBS_ERR_SHAPE, "pbs_gemm: NVFP4 needs K %% 128 == 0");
      PBS_REQUIRE(((uintptr_t)a_scale & 3) == 0 && ((uintptr_t)b_scale & 3) == 0, PBS_ERR_INVALID_ARG,
                  "pbs_gemm: NVFP4 block scales must be 4-byte aligned");
      g.lda = K / 2; g.ldb = K / 2;
      if (bf16_out) fn = w2d ? gemm_nvfp4_kernel<true, true> : gemm_nvfp4_kernel<false, true>;
      else fn = w2d ? gemm_nvfp4_kernel<true, false> : gemm_nvfp4_kernel<false, false>;
      name = "gemm_nvfp4";
      break;
    }
    default:
      return set_error(PBS_ERR_INVALID_ARG, "pbs_gemm: unknown recipe %d", (int)recipe);
  }
  // tiles address their 256 rows with 32-bit offsets: stored rows up to 16 MiB
  PBS_REQUIRE(g.lda <= (1 << 24) && g.ldb <= (1 << 24), PBS_ERR_SHAPE,
              "pbs_gemm: stored operand rows longer than 16 MiB are not supported");
  const unsigned grid = (unsigned)(g.tiles_m * g.tiles_n);
  log_dispatch("%s layout=%d M=%lld N=%lld K=%lld out=%s tiles=%dx%d", name, (int)layout, (long long)M,
               (long long)N, (long long)K, bf16_out ? "bf16" : "f32", g.tiles_m, g.tiles_n);
  if (c_amax) hipLaunchKernelGGL(zero_word_kernel, dim3(1), dim3(64), 0, stream, (uint32_t*)c_amax);
  hipLaunchKernelGGL(fn, dim3(grid), dim3(nthr), 0, stream, g);
  return check_launch("pbs_gemm");
}

extern "C" pbs_status pbs_gemm(pbs_recipe recipe, pbs_layout layout, int64_t M, int64_t N, int64_t K,
                               const void* A, pbs_format a_fmt, const void* a_scale,
                               const float* a_tensor_scale, const void* B, pbs_format b_fmt,
                               const void* b_scale, const float* b_tensor_scale, void* C,
                               pbs_format c_fmt, hipStream_t stream) {
  return gemm_impl(recipe, layout, M, N, K, A, a_fmt, a_scale, a_tensor_scale, B, b_fmt, b_scale,
                   b_tensor_scale, C, c_fmt, nullptr, stream);
}

extern "C" pbs_status pbs_gemm_amax(pbs_recipe recipe, pbs_layout layout, int64_t M, int64_t N, int64_t K,
                                    const void* A, pbs_format a_fmt, const void* a_scale,
                                    const float* a_tensor_scale, const void* B, pbs_format b_fmt,
                                    const void* b_scale, const float* b_tensor_scale, void* C,
                                    pbs_format c_fmt, float* c_amax, hipStream_t stream) {
  PBS_REQUIRE(c_amax, PBS_ERR_INVALID_ARG, "pbs_gemm_amax: c_amax is null");
  PBS_REQUIRE(((uintptr_t)c_amax & 3) == 0, PBS_ERR_INVALID_ARG, "pbs_gemm_amax: c_amax not 4-byte aligned");
  return gemm_impl(recipe, layout, M, N, K, A, a_fmt, a_scale, a_tensor_scale, B, b_fmt, b_scale,
                   b_tensor_scale, C, c_fmt, c_amax, stream);
}
