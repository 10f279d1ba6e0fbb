// Pieces shared by the GEMM kernels (gemm.hip, gemm_blk.hip): vector
// types, the kernel argument block, the swizzled LDS tile layout, operand
// and scale-row staging straight into LDS, and the XCD-aware tile order.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pbs {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256, NTHR = 256;     // tile rows per workgroup, threads per workgroup
constexpr int ROWB = 128;               // bytes per LDS row per K stage
constexpr int TILEB = BM * ROWB;        // 32 KB per 256-row operand tile per stage
constexpr int GROUP_M = 4;              // tile rows walked together (L2 reuse; 4 measured best of 1-32)
constexpr int NXCD = 8;
constexpr int cmax(int a, int b) { return a > b ? a : b; }

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
  int tiles_m, tiles_n;
  int a_sdiv, b_sdiv;     // MX scale rows: operand rows per stored scale row (1, or 128 for 128x128 blocks)
  uint32_t* c_amax;       // optional: max |C| of the stored output (fp32 bits), folded in by the epilogue
};

// max |x| of the 8 bf16 / 4 fp32 values of a stored 16-byte chunk of C, as
// fp32 bits (for non-negative IEEE values bit order is numeric order).
__device__ __forceinline__ uint32_t absmax_bf16x8(uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = (w[i] & 0x7FFFu) << 16, hi = w[i] & 0x7FFF0000u;
    m = m > lo ? m : lo;
    m = m > hi ? m : hi;
  }
  return m;
}

__device__ __forceinline__ uint32_t absmax_f32x4(uint4 v) {
  const uint32_t w[4] = {v.x & 0x7FFFFFFFu, v.y & 0x7FFFFFFFu, v.z & 0x7FFFFFFFu, v.w & 0x7FFFFFFFu};
  const uint32_t a = w[0] > w[1] ? w[0] : w[1], b = w[2] > w[3] ? w[2] : w[3];
  return a > b ? a : b;
}

// Fold a per-lane maximum into *out: wave reduction, the workgroup's NW
// waves through the first 4 NW bytes of the (finished) epilogue staging area,
// then one atomic from thread 0 only when the workgroup's maximum exceeds
// what *out already holds.  Thousands of same-address atomics queue behind
// each other, so there is at most one per workgroup.  No LDS object of its
// own: a second one in the kernel makes the compiler wait for every LDS DMA
// load in flight before each LDS read of the main loop.  Called by all
// threads of the workgroup after its last read of `smem` (two barriers).
template <int NW = NTHR / 64>
__device__ __forceinline__ void amax_fold_wg(uint32_t v, uint32_t* out, uint8_t* smem) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t u = (uint32_t)__shfl_xor((int)v, o, 64);
    v = v > u ? v : u;
  }
  uint32_t* part = (uint32_t*)smem;
  __syncthreads();                                   // every wave is done with the staging area
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = part[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) m = m > part[i] ? m : part[i];
    const uint32_t cur = __builtin_nontemporal_load(out);
    if (m > cur) atomicMax(out, m);
  }
}

// LDS tile layout: row r, 16-byte chunk c lives at r * 128 + ((c ^ key(r)) << 4).
// gfx950's LDS serves a 16-byte-per-lane access 16 lanes (256 bytes, 64
// banks) at a time; key(r) = (r ^ r >> 1 ^ r >> 4) & 7 makes the MFMA
// fragment reads (16 consecutive rows, one chunk) conflict-free, and the
// MN-major bf16 stores at most 2-way (a plain
// r & 7 leaves every fragment read 2-way conflicted).
__device__ __forceinline__ int swz_key(int row) { return (row ^ (row >> 1) ^ (row >> 4)) & 7; }
__device__ __forceinline__ int swz(int row, int chunk) { return row * ROWB + ((chunk ^ swz_key(row)) << 4); }

__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---------------------------------------------------------------------------
// Operand staging.  Every variant fills one [256 rows][128 B] swizzled LDS
// tile for K stage kt.  rows0 / nrows: first tile row and valid rows (rows
// past the end re-read the last valid row; their results are never stored).
// ---------------------------------------------------------------------------

// K-major, direct to LDS (buffer_load_dwordx4 ... lds, no registers): load i
// (of 8) of wave w fills LDS rows 64 w + 8 i .. + 7; lane l owns row
// 64 w + 8 i + l / 8, physical chunk l % 8, i.e. the logical chunk that the
// swizzle places there.  The tile's rows are one buffer resource (base = its
// first row, range = the bytes to the operand's end, at most 2^32 - 1), so a
// load is that resource, the lane's 32-bit offset and the stage's byte offset
// in a scalar register: no per-lane 64-bit address arithmetic (row * ld <
// 2^32 is checked on the host).
struct Direct {
  __amdgpu_buffer_rsrc_t r;
  uint32_t off[8];
};

constexpr int BUF_RSRC_WORD3 = 0x00020000;   // raw, untyped gfx9 buffer (32-bit data format field)

__device__ __forceinline__ void direct_init(Direct& d, const uint8_t* p, int64_t ld, int rows0, int nrows,
                                            int w) {
  const int lane = threadIdx.x & 63;
  const int64_t span = (int64_t)(nrows - rows0) * ld;
  d.r = __builtin_amdgcn_make_buffer_rsrc((void*)(p + (int64_t)rows0 * ld), (short)0,
                                          (int)(uint32_t)(span < 0xFFFFFFFFll ? span : 0xFFFFFFFFll), BUF_RSRC_WORD3);
  const int lim = nrows - rows0 - 1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int trow = 64 * w + 8 * i + (lane >> 3);
    const int lc = (lane & 7) ^ swz_key(trow);
    const int r = trow < lim ? trow : lim;
    d.off[i] = (uint32_t)r * (uint32_t)ld + (uint32_t)(lc << 4);
  }
}

__device__ __forceinline__ void direct_item(const Direct& d, int kt, uint8_t* tile, int w, int i) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(d.r, (lds_ptr_t)(tile + (w * 8 + i) * 1024), 16, d.off[i],
                                           (uint32_t)(kt * ROWB), 0, 0);
}

// One dword per tile row per stage (MX scales: 4 E8M0 bytes; block-128: one
// fp32 scale), direct to LDS: wave w loads rows 64 w .. 64 w + 63.
struct RowDword {
  const uint8_t* p;        // this lane's row of the scale array
};

__device__ __forceinline__ void rowdw_init(RowDword& d, const uint8_t* scale, int64_t row_stride, int rows0,
                                           int nrows, int div_rows, int w) {
  const int lane = threadIdx.x & 63;
  int row = rows0 + 64 * w + lane;
  row = row < nrows ? row : nrows - 1;
  d.p = scale + (int64_t)(row / div_rows) * row_stride;
}

__device__ __forceinline__ void rowdw_issue(const RowDword& d, int kt, uint32_t* ring_slot, int w) {
  __builtin_amdgcn_global_load_lds(d.p + (int64_t)kt * 4, (lds_ptr_t)(ring_slot + 64 * w), 4, 0, 0);
}

// XCD-aware tile order: workgroup b runs on XCD b % 8; give each XCD a
// contiguous range of logical tiles, then walk tiles GROUP_M rows at a time.
__device__ __forceinline__ void tile_of(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n;
  const int q = T / NXCD, r = T % NXCD;
  const int x = b % NXCD, idx = b / NXCD;
  const int id = x * q + (x < r ? x : r) + idx;
  const int per_group = GROUP_M * tiles_n;
  const int g = id / per_group;
  const int first_m = g * GROUP_M;
  const int gm = (tiles_m - first_m) < GROUP_M ? (tiles_m - first_m) : GROUP_M;
  const int in = id - g * per_group;
  tm = first_m + in % gm;
  tn = in / gm;
}

__device__ __forceinline__ i32x8 read2(const uint8_t* tile_row0, uint32_t lb, uint32_t x) {
  const i32x4 lo = *(const i32x4*)(tile_row0 + (lb ^ x));
  const i32x4 hi = *(const i32x4*)(tile_row0 + (lb ^ x ^ 32u));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

typedef void (*gemm_fn)(GemmArgs);

// Sub-channel (block-128) FP8 kernel of gemm_blk.hip: 128x128 (a2d / b2d)
// or 1x128 blocks for A and B (a2d implies b2d), bf16 or fp32 output;
// BLK_THR threads per workgroup, BM x BLK_BN output tiles.
constexpr int BLK_THR = 512, BLK_BN = 256;
gemm_fn blk_kernel_for(bool a2d, bool b2d, bool bf16_out);

}  // namespace pbs
