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

// Exclusive scan of in[0, n) into out[0, n], out[n] = the total (also written
// to *total_out when given), by one workgroup of NT threads; every thread calls
// it. Items are held blocked, I per thread per tile of NT * I items, and the
// next tile's loads are issued before the current tile is scanned.
template <typename T, int NT, int I>
__device__ __forceinline__ void block_scan_all(const T* in, T* out, int64_t n, T* total_out, T* s_wave) {
  constexpr int64_t kTile = (int64_t)NT * I;
  const int64_t tb = (int64_t)threadIdx.x * I;
  T v[I];
#pragma unroll
  for (int k = 0; k < I; ++k) v[k] = tb + k < n ? in[tb + k] : T(0);
  T carry = 0;
  for (int64_t c = 0; c < n; c += kTile) {  // uniform
    T nx[I];
    const int64_t nb = c + kTile + tb;
#pragma unroll
    for (int k = 0; k < I; ++k) nx[k] = nb + k < n ? in[nb + k] : T(0);
    T sum = 0;
#pragma unroll
    for (int k = 0; k < I; ++k) sum += v[k];
    T total;
    T excl = block_excl_scan<T, NT>(sum, s_wave, total) + carry;
#pragma unroll
    for (int k = 0; k < I; ++k) {
      const int64_t i = c + tb + k;
      if (i < n) out[i] = excl;
      excl += v[k];
      v[k] = nx[k];
    }
    carry += total;
  }
  if (threadIdx.x == 0) {
    out[n] = carry;
    if (total_out) *total_out = carry;
  }
}

__device__ __forceinline__ int popc64(uint64_t x) { return __popcll(x); }

// Voxel counts of a 256-thread block's leaves (v = 0 on lanes that own no leaf):
// returns this thread's exclusive prefix inside the block and writes the block's
// total to *total_dst. Every thread of the block must call it (block barriers).
__device__ __forceinline__ int32_t block_run_scan(int32_t v, int64_t* total_dst) {
  __shared__ int32_t s_wave[4];
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  int32_t inc = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int32_t t = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += t;
  }
  if (lane == kWave - 1) s_wave[w] = inc;
  __syncthreads();
  int32_t off = 0;
  for (int i = 0; i < w; ++i) off += s_wave[i];
  if (threadIdx.x == 0) *total_dst = (int64_t)s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
  return off + inc - v;
}

// Workgroups are dispatched round-robin over the chip's 8 XCDs (workgroup b on
// XCD b % 8), and each XCD has its own L2. Logical block of dispatched block b
// out of nb: XCD x takes the contiguous range of about nb / 8 logical blocks
// starting at x * (nb / 8) + min(x, nb % 8), so neighbouring work items, which
// read the same source data, share one L2. A bijection on [0, nb).
__device__ __forceinline__ int64_t xcd_block(int64_t b, int64_t nb) {
  constexpr int64_t kXcds = 8;
  const int64_t q = nb / kXcds, r = nb % kXcds, x = b % kXcds;
  return x * q + (x < r ? x : r) + b / kXcds;
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

// Quads (4 consecutive lanes): lane q of a quad reads lane p_q of the same
// quad (DPP quad permutation, no old value: one instruction). A DPP read from a
// lane that EXEC disables is undefined, so the permutation must run with the
// whole quad active: the empty volatile asm on its result keeps the compiler
// from moving it into a branch taken by part of the quad (it would otherwise
// fold `cond ? x : perm(y)` into a perm executed only by the lanes where cond
// is false). Call it from code every lane of the quad executes.
template <int p0, int p1, int p2, int p3>
__device__ __forceinline__ int quad_perm32(int v) {
  int r = __builtin_amdgcn_mov_dpp(v, p0 | (p1 << 2) | (p2 << 4) | (p3 << 6), 0xf, 0xf, false);
  asm volatile("" : "+v"(r));
  return r;
}
template <int p0, int p1, int p2, int p3>
__device__ __forceinline__ uint64_t quad_perm64(uint64_t v) {
  const uint32_t lo = (uint32_t)quad_perm32<p0, p1, p2, p3>((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)quad_perm32<p0, p1, p2, p3>((int)(uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
template <int k>  // lane k of the quad, to all four
__device__ __forceinline__ int quad_bcast32(int v) {
  return quad_perm32<k, k, k, k>(v);
}
// As quad_bcast32 with k known only after unrolling (k must fold to a constant).
__device__ __forceinline__ int quad_bcast32(int v, int k) {
  switch (k & 3) {
    case 0: return quad_bcast32<0>(v);
    case 1: return quad_bcast32<1>(v);
    case 2: return quad_bcast32<2>(v);
    default: return quad_bcast32<3>(v);
  }
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

// Bit k of the result is set when byte k of w (8 bytes) is non-zero.
__device__ __forceinline__ uint32_t nonzero_bytes(uint64_t w) {
  uint32_t m = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t x = (uint32_t)(w >> (32 * h));
    uint32_t t = (((x & 0x7f7f7f7fu) + 0x7f7f7f7fu) | x) & 0x80808080u;  // top bit of a non-zero byte
    t >>= 7;                                                             // bits 0, 8, 16, 24
    t = (t | (t >> 7) | (t >> 14) | (t >> 21)) & 0xfu;
    m |= t << (4 * h);
  }
  return m;
}

__device__ __forceinline__ void leaf_stats(const uint64_t W[8], uint64_t& prefix, int& count, uint32_t& box) {
  uint64_t packed = 0, orw = 0;
  uint32_t run = 0, nzw = 0;  // running popcount; non-empty words (bit k: word k = x)
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k > 0) packed |= (uint64_t)run << (9 * (k - 1));
    run += (uint32_t)__popcll(W[k]);
    nzw |= (W[k] != 0 ? 1u : 0u) << k;
    orw |= W[k];
  }
  prefix = packed;
  count = (int)run;
  if (!orw) {
    box = kEmptyBox;
    return;
  }
  // y extent: non-zero bytes of the OR of all words; z extent: OR of those bytes
  const uint32_t nzy = nonzero_bytes(orw);
  uint32_t zor = (uint32_t)orw | (uint32_t)(orw >> 32);
  zor |= zor >> 16;
  zor = (zor | (zor >> 8)) & 0xffu;
  const int xmin = __builtin_ctz(nzw), xmax = 31 - __builtin_clz(nzw);
  const int ymin = __builtin_ctz(nzy), ymax = 31 - __builtin_clz(nzy);
  const int zmin = __builtin_ctz(zor), zmax = 31 - __builtin_clz(zor);
  box = (uint32_t)(xmin | (xmax << 3) | (ymin << 6) | (ymax << 9) | (zmin << 12) | (zmax << 15));
}

// leaf_stats for a leaf whose 8 words are spread over a quad (lane s of the
// quad holds words 2s and 2s+1): the same prefix word, count and packed box,
// on every lane of the quad. `sub` is the lane's index in the quad.
__device__ __forceinline__ void quad_leaf_stats(uint64_t w0, uint64_t w1, int sub, uint64_t& prefix, int& count,
                                                uint32_t& box) {
  const int c0 = __popcll(w0), cs = c0 + __popcll(w1);
  int inc = cs;  // inclusive scan of the lanes' counts over the quad
  {
    const int t = quad_perm32<0, 0, 1, 2>(inc);
    if (sub >= 1) inc += t;
  }
  {
    const int t = quad_perm32<0, 0, 0, 1>(inc);
    if (sub >= 2) inc += t;
  }
  const int ex = inc - cs;  // voxels in words < 2 sub
  count = quad_bcast32<3>(inc);
  // field w-1 (9 bits each) = voxels in words < w: this lane's w = 2 sub + 1 and w = 2 sub
  uint64_t pf = (uint64_t)(ex + c0) << (18 * sub);
  if (sub > 0) pf |= (uint64_t)ex << (18 * sub - 9);
  pf |= quad_perm64<1, 0, 3, 2>(pf);
  pf |= quad_perm64<2, 3, 0, 1>(pf);
  prefix = pf;
  int xmin = w0 ? 2 * sub : (w1 ? 2 * sub + 1 : 8);
  int xmax = w1 ? 2 * sub + 1 : (w0 ? 2 * sub : -1);
  xmin = min(xmin, quad_perm32<1, 0, 3, 2>(xmin));
  xmin = min(xmin, quad_perm32<2, 3, 0, 1>(xmin));
  xmax = max(xmax, quad_perm32<1, 0, 3, 2>(xmax));
  xmax = max(xmax, quad_perm32<2, 3, 0, 1>(xmax));
  uint64_t orw = w0 | w1;
  orw |= quad_perm64<1, 0, 3, 2>(orw);
  orw |= quad_perm64<2, 3, 0, 1>(orw);
  if (!orw) {
    box = kEmptyBox;
    return;
  }
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
