// Device-side helpers: wave64 scans and reductions, bit tricks.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tc {

constexpr int kWave = 64;

template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    T n = __shfl_up(v, d, kWave);
    if (lane >= d) v += n;
  }
  return v;
}

// Exclusive block scan for NT threads (NT a multiple of 64). `s_wave` holds
// NT/64 entries of shared memory. Returns the exclusive prefix and the total.
template <typename T, int NT>
__device__ __forceinline__ T block_excl_scan(T v, T* s_wave, T& total) {
  const int w = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  T inc = wave_incl_scan(v);
  if (lane == kWave - 1) s_wave[w] = inc;
  __syncthreads();
  T off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) {
    T x = s_wave[i];
    if (i < w) off += x;
    tot += x;
  }
  __syncthreads();
  total = tot;
  return off + inc - v;
}

__device__ __forceinline__ int popc64(uint64_t x) { return __popcll(x); }

// Sum of v over a 256-thread block, written to *dst by thread 0. Every thread of
// the block must call it (it holds a block barrier).
__device__ __forceinline__ void block_sum_to(int64_t v, int64_t* dst) {
  __shared__ int64_t s_part[4];
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0) s_part[threadIdx.x / kWave] = v;
  __syncthreads();
  if (threadIdx.x == 0) *dst = s_part[0] + s_part[1] + s_part[2] + s_part[3];
}

// Index of the r-th set bit (0-based) of w; w must have more than r set bits.
__device__ __forceinline__ int select_bit(uint64_t w, int r) {
  int pos = 0;
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    const uint64_t low = (s == 64) ? ~0ull : ((1ull << s) - 1);
    const int c = __popcll(w & low);
    if (r >= c) {
      r -= c;
      w >>= s;
      pos += s;
    }
  }
  return pos;
}

__device__ __forceinline__ int wave_min_i32(int v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = min(v, __shfl_xor(v, d, kWave));
  return v;
}
__device__ __forceinline__ int wave_max_i32(int v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = max(v, __shfl_xor(v, d, kWave));
  return v;
}

// Statistics of a final leaf mask W (bit n = x*64 + y*8 + z):
//   prefix  seven 9-bit fields, field w-1 = voxels in words < w
//   count   voxels in the leaf
//   box     local bbox packed as xmin | xmax<<3 | ymin<<6 | ymax<<9 | zmin<<12 |
//           zmax<<15 (3 bits each); kEmptyBox for an empty mask
constexpr uint32_t kEmptyBox = 0xffffffffu;

__device__ __forceinline__ void leaf_stats(const uint64_t W[8], uint64_t& prefix, int& count, uint32_t& box) {
  uint64_t packed = 0, run = 0, orw = 0;
  int xmin = 8, xmax = -1;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k > 0) packed |= run << (9 * (k - 1));
    run += (uint64_t)__popcll(W[k]);
    if (W[k]) {
      xmin = min(xmin, k);
      xmax = max(xmax, k);
    }
    orw |= W[k];
  }
  prefix = packed;
  count = (int)run;
  if (!orw) {
    box = kEmptyBox;
    return;
  }
  // y extent: non-zero bytes of the OR of all words; z extent: OR of those bytes
  int ymin = 8, ymax = -1;
  uint64_t zor = 0;
#pragma unroll
  for (int y = 0; y < 8; ++y) {
    const uint64_t byte = (orw >> (8 * y)) & 0xffull;
    if (byte) {
      ymin = min(ymin, y);
      ymax = max(ymax, y);
    }
    zor |= byte;
  }
  const int zmin = __builtin_ctzll(zor);
  const int zmax = 63 - __builtin_clzll(zor);
  box = (uint32_t)(xmin | (xmax << 3) | (ymin << 6) | (ymax << 9) | (zmin << 12) | (zmax << 15));
}

}  // namespace tc
