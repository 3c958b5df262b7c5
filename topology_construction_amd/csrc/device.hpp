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

}  // namespace tc
