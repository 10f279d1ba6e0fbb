// Per-tensor amax, scale derivation and the delayed-scaling history.
//
// amax: "Optimizing Transformer models for low-precision training",
// "Technical deep-dive" (per-tensor scale from the max absolute value);
// "How to optimize Transformer-based models for low-precision training",
// "Interpreting results for a real model" (NVFP4 needs an extra memory pass
// for the per-tensor maximum, taken after the random Hadamard transform on
// the Wgrad inputs).
//
// The reduction is over magnitudes as unsigned integers: for non-negative
// IEEE values, bit-pattern order is numeric order, so a bf16 max is a
// 16-bit integer max of (bits & 0x7FFF) and the fp32 result is those bits
// shifted up.  Max is order-independent, so the result is deterministic.
#include "device.hpp"
#include "host.hpp"

#include <algorithm>

namespace pbs {

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint32_t w = (uint32_t)__shfl_xor((int)v, o, 64);
    v = v > w ? v : w;
  }
  return v;
}

// Block-wide max of a per-thread value, then at most one atomic max per
// block: only when the block's maximum exceeds what *out already holds (the
// running maximum settles early, so most blocks skip the same-address
// atomic, which would otherwise serialize thousands of blocks at the end).
__device__ __forceinline__ void block_max_atomic(uint32_t v, uint32_t* out) {
  __shared__ uint32_t part[16];
  v = wave_max_u32(v);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) part[wid] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = 0;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) m = m > part[i] ? m : part[i];
    const uint32_t cur = __builtin_nontemporal_load(out);
    if (m > cur) atomicMax(out, m);
  }
}

__global__ void fill_u32_kernel(uint32_t* p, uint32_t v) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *p = v;
}

// Plain amax over n bf16 values; n8 = n / 8 full 16-byte chunks, the rest
// (n % 8 values) handled by block 0.  Each block reads 32 KB contiguous per
// iteration (chunks [(j * grid + b) * 2048, + 2048): thread t takes chunks
// t, t + 256, ... of them, eight 16-byte loads in flight before any
// arithmetic).  Measured on a 1 GiB read: 7.0 TB/s with this block-contiguous
// order against 5.6-6.0 TB/s when consecutive blocks interleave their 4 KB
// pieces (grid-stride order); 1024-16384 blocks all within 1%.  Chunks past
// the end re-read the last one (harmless for a maximum).
__global__ __launch_bounds__(256) void amax_bf16_kernel(const uint4* __restrict__ x, int64_t n8,
                                                        const bf16_t* __restrict__ tail, int tail_n,
                                                        uint32_t* out) {
  constexpr int U = 8;
  us2 m = {0, 0};
  const us2 mask = {0x7FFF, 0x7FFF};
  const int64_t span = 256 * U;
  for (int64_t base = (int64_t)blockIdx.x * span; base < n8; base += (int64_t)gridDim.x * span) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int64_t j = base + u * 256 + threadIdx.x;
      j = j < n8 ? j : n8 - 1;
      v[u] = ld_nt16(&x[j]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, v[u].x) & mask);
      m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, v[u].y) & mask);
      m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, v[u].z) & mask);
      m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, v[u].w) & mask);
    }
  }
  uint32_t mm = m.x > m.y ? m.x : m.y;
  if (blockIdx.x == 0 && (int)threadIdx.x < tail_n) {
    uint32_t t = tail[threadIdx.x] & 0x7FFFu;
    mm = mm > t ? mm : t;
  }
  block_max_atomic(mm << 16, out);
}

// amax of the RHT16 output along the rows: one work item = one group of 16
// rows x 8 columns (sixteen 16-byte loads, coalesced across the wave).  The
// transform's arithmetic is trimmed to what the maximum needs, with the same
// result bit for bit: the sign flips go onto the packed bf16 words (both
// values of a word are in one row, so they share sigma_r), and the exact
// multiply by 1/4 is applied once to the final maximum -- rounding x / 4 is
// monotone in |x|, so the maximum of the rounded values is the rounding of
// the maximum.
__global__ __launch_bounds__(256) void amax_rht_kernel(const bf16_t* __restrict__ x, int64_t rows,
                                                       int64_t cols, uint64_t seed, uint32_t* out) {
  __shared__ uint32_t s_mask;
  if (threadIdx.x < 64) {
    uint32_t bit = 0;
    if (threadIdx.x < 16)
      bit = philox_word0(threadIdx.x, 0u, 1u, 0u, (uint32_t)seed, (uint32_t)(seed >> 32)) & 1u;
    uint64_t b = __ballot(bit);
    if (threadIdx.x == 0) s_mask = (uint32_t)b;
  }
  __syncthreads();
  const uint32_t sign_mask = __builtin_amdgcn_readfirstlane(s_mask);
  const int64_t c8n = cols / 8;
  const int64_t items = (rows / 16) * c8n;
  uint32_t m = 0;
  for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < items;
       it += (int64_t)gridDim.x * blockDim.x) {
    const int64_t g = it / c8n, c8 = it - g * c8n;
    const bf16_t* p = x + (g * 16) * cols + c8 * 8;
    uint4 v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = ld_nt16(p + r * cols);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t sx = ((sign_mask >> r) & 1u) ? 0x80008000u : 0u;
      v[r].x ^= sx;
      v[r].y ^= sx;
      v[r].z ^= sx;
      v[r].w ^= sx;
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float u[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t w = (c < 2) ? v[r].x : (c < 4) ? v[r].y : (c < 6) ? v[r].z : v[r].w;
        u[r] = __uint_as_float((c & 1) ? (w & 0xFFFF0000u) : (w << 16));
      }
#pragma unroll
      for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if ((i & h) == 0) {
            const float a = u[i], b = u[i + h];
            u[i] = a + b;
            u[i + h] = a - b;
          }
        }
      }
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const uint32_t a = __float_as_uint(u[r]) & 0x7FFFFFFFu, b = __float_as_uint(u[r + 1]) & 0x7FFFFFFFu;
        const uint32_t ab = a > b ? a : b;
        m = m > ab ? m : ab;
      }
    }
  }
  // the 1/4 of the transform, on the maximum (inf stays inf; NaN bits stay NaN)
  m = __float_as_uint(__uint_as_float(m) * 0.25f) & 0x7FFFFFFFu;
  block_max_atomic(m, out);
}

__global__ void scale_from_amax_kernel(const float* amax, float fmax, float* scale, float* scale_inv) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  float s = scale_from_amax(*amax, fmax);
  if (scale) *scale = s;
  if (scale_inv) *scale_inv = 1.0f / s;
}

// Delayed-scaling state: {float scale; float scale_inv; int32 pos; int32 len; float hist[len]}.
struct DelayedHeader {
  float scale;
  float scale_inv;
  int32_t pos;
  int32_t len;
};

__global__ void delayed_init_kernel(DelayedHeader* st, int len) {
  float* hist = (float*)(st + 1);
  for (int i = threadIdx.x; i < len; i += blockDim.x) hist[i] = 0.0f;
  if (threadIdx.x == 0) {
    st->scale = 1.0f;
    st->scale_inv = 1.0f;
    st->pos = 0;
    st->len = len;
  }
}

// One wave: push amax into the ring, new scale from the ring's maximum.
__global__ void delayed_update_kernel(DelayedHeader* st, const float* amax, float fmax) {
  float* hist = (float*)(st + 1);
  const int len = st->len;
  const int pos = st->pos;
  const float a = *amax;
  uint32_t m = 0;
  for (int i = threadIdx.x; i < len; i += 64) {
    float h = (i == pos) ? a : hist[i];
    uint32_t hb = __float_as_uint(h);
    m = m > hb ? m : hb;
  }
  m = wave_max_u32(m);
  __syncthreads();
  if (threadIdx.x == 0) {
    hist[pos] = a;
    st->pos = (pos + 1) % len;
    float s = scale_from_amax(__uint_as_float(m), fmax);
    st->scale = s;
    st->scale_inv = 1.0f / s;
  }
}

static int amax_grid(int64_t work_items, int per_thread) {
  int64_t blocks = ceil_div(work_items, (int64_t)256 * per_thread);
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  return (int)blocks;
}

}  // namespace pbs

using namespace pbs;

extern "C" {

pbs_status pbs_amax(const void* x_bf16, int64_t rows, int64_t cols, int flags, uint64_t seed,
                    float* amax_out, hipStream_t stream) {
  PBS_REQUIRE(amax_out, PBS_ERR_INVALID_ARG, "pbs_amax: amax_out is null");
  PBS_REQUIRE(rows >= 0 && cols >= 0, PBS_ERR_SHAPE, "pbs_amax: negative shape");
  PBS_REQUIRE((flags & ~PBS_FLAG_RHT16) == 0, PBS_ERR_INVALID_ARG, "pbs_amax: unknown flags %d", flags);
  const int64_t n = rows * cols;
  PBS_REQUIRE(n == 0 || x_bf16, PBS_ERR_INVALID_ARG, "pbs_amax: x is null");
  uint32_t* out = (uint32_t*)amax_out;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(64), 0, stream, out, 0u);
  if (n == 0) return check_launch("pbs_amax");
  if (flags & PBS_FLAG_RHT16) {
    PBS_REQUIRE(rows % 16 == 0 && cols % 8 == 0, PBS_ERR_SHAPE,
                "pbs_amax: RHT16 needs rows %% 16 == 0 and cols %% 8 == 0 (got %lld x %lld)",
                (long long)rows, (long long)cols);
    PBS_REQUIRE(((uintptr_t)x_bf16 & 15) == 0, PBS_ERR_INVALID_ARG, "pbs_amax: x not 16-byte aligned");
    int grid = std::min(amax_grid((rows / 16) * (cols / 8), 2), 1024);   // one atomic per block
    log_dispatch("amax_rht_kernel rows=%lld cols=%lld grid=%d", (long long)rows, (long long)cols, grid);
    hipLaunchKernelGGL(amax_rht_kernel, dim3(grid), dim3(256), 0, stream, (const bf16_t*)x_bf16,
                       rows, cols, seed, out);
  } else {
    PBS_REQUIRE(((uintptr_t)x_bf16 & 15) == 0, PBS_ERR_INVALID_ARG, "pbs_amax: x not 16-byte aligned");
    const int64_t n8 = n / 8;
    const int tail_n = (int)(n - n8 * 8);
    // at most 1024 blocks: one same-address atomic per block at the end, so
    // fewer, longer-lived blocks (1024 read as fast as 4096 in a probe)
    int grid = std::min(amax_grid(n8, 32), 1024);
    log_dispatch("amax_bf16_kernel n=%lld grid=%d", (long long)n, grid);
    hipLaunchKernelGGL(amax_bf16_kernel, dim3(grid), dim3(256), 0, stream, (const uint4*)x_bf16, n8,
                       (const bf16_t*)x_bf16 + n8 * 8, tail_n, out);
  }
  return check_launch("pbs_amax");
}

pbs_status pbs_scale_from_amax(const float* amax, float fmax, float* scale, float* scale_inv,
                               hipStream_t stream) {
  PBS_REQUIRE(amax, PBS_ERR_INVALID_ARG, "pbs_scale_from_amax: amax is null");
  PBS_REQUIRE(fmax > 0.0f, PBS_ERR_INVALID_ARG, "pbs_scale_from_amax: fmax must be > 0");
  hipLaunchKernelGGL(scale_from_amax_kernel, dim3(1), dim3(64), 0, stream, amax, fmax, scale, scale_inv);
  return check_launch("pbs_scale_from_amax");
}

pbs_status pbs_delayed_state_bytes(int hist_len, size_t* bytes) {
  PBS_REQUIRE(bytes, PBS_ERR_INVALID_ARG, "pbs_delayed_state_bytes: bytes is null");
  PBS_REQUIRE(hist_len >= 1 && hist_len <= 4096, PBS_ERR_INVALID_ARG,
              "pbs_delayed_state_bytes: hist_len must be in [1, 4096]");
  *bytes = sizeof(DelayedHeader) + (size_t)hist_len * sizeof(float);
  return PBS_OK;
}

pbs_status pbs_delayed_init(void* state, int hist_len, hipStream_t stream) {
  PBS_REQUIRE(state, PBS_ERR_INVALID_ARG, "pbs_delayed_init: state is null");
  PBS_REQUIRE(hist_len >= 1 && hist_len <= 4096, PBS_ERR_INVALID_ARG,
              "pbs_delayed_init: hist_len must be in [1, 4096]");
  hipLaunchKernelGGL(delayed_init_kernel, dim3(1), dim3(256), 0, stream, (DelayedHeader*)state, hist_len);
  return check_launch("pbs_delayed_init");
}

pbs_status pbs_delayed_update(void* state, const float* amax, float fmax, hipStream_t stream) {
  PBS_REQUIRE(state && amax, PBS_ERR_INVALID_ARG, "pbs_delayed_update: null pointer");
  PBS_REQUIRE(fmax > 0.0f, PBS_ERR_INVALID_ARG, "pbs_delayed_update: fmax must be > 0");
  hipLaunchKernelGGL(delayed_update_kernel, dim3(1), dim3(64), 0, stream, (DelayedHeader*)state, amax, fmax);
  return check_launch("pbs_delayed_update");
}

float* pbs_delayed_scale(void* state) { return state ? &((DelayedHeader*)state)->scale : nullptr; }
float* pbs_delayed_scale_inv(void* state) { return state ? &((DelayedHeader*)state)->scale_inv : nullptr; }

}  // extern "C"
