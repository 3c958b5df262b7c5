// Data-parallel primitives for gfx950: exclusive scans, fills and a 128-bit-key
// sort (single-workgroup bitonic for small inputs, LSD radix with 8-bit digits and
// wave64 ballot ranking otherwise). These serve the node-level stages of the
// topology pass; the leaf-level work never goes through a sort.
#include "device.hpp"
#include "internal.hpp"

namespace tc {

constexpr int kScanThreads = 256;
constexpr int kScanItems = 16;
constexpr int kScanTile = kScanThreads * kScanItems;  // 4096

__device__ __forceinline__ i64 clamp_n(i64 n_host, const int32_t* d_n) {
  i64 n = d_n ? (i64)(*d_n) : n_host;
  if (n > n_host) n = n_host;
  if (n < 0) n = 0;
  return n;
}

// In the multi-block scan a tile of kScanTile items is held striped: item
// k * kScanThreads + t in register k of thread t, so every load and store
// instruction is coalesced. The tile's
// exclusive scan is a wave scan per row k plus one 64-entry table of the
// (row, wave) totals, scanned by one wave.
static_assert(kScanItems * (kScanThreads / kWave) == kWave, "one table entry per lane");

template <typename T>
__device__ __forceinline__ T tile_scan_striped(const T v[kScanItems], T ex[kScanItems], T* s_tab) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  T inc[kScanItems];
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) {
    inc[k] = wave_incl_scan(v[k]);
    if (lane == kWave - 1) s_tab[k * (kScanThreads / kWave) + w] = inc[k];
  }
  __syncthreads();
  if (w == 0) {
    const T t = s_tab[lane];
    const T i2 = wave_incl_scan(t);
    s_tab[lane] = i2 - t;
    if (lane == kWave - 1) s_tab[kWave] = i2;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) ex[k] = s_tab[k * (kScanThreads / kWave) + w] + inc[k] - v[k];
  const T total = s_tab[kWave];
  __syncthreads();  // the table is free again
  return total;
}

// Single-workgroup scans (up to kScanSingleMax items, one workgroup of NT
// threads) hold items blocked: thread t owns items t*I .. +I-1 of the current
// tile of NT I items (I = 16, or 8 for 8-byte items in 1024-thread workgroups
// so that the next tile's registers fit beside the current one's), which needs
// one block scan per tile; the next tile's loads are issued before the current
// one is scanned. These launches are latency-bound, so fewer steps (and one
// launch instead of three) beat coalescing: scans of more than kScanSingleWide
// items take a 1024-thread workgroup (fewer steps), smaller ones 256 threads
// (a shorter launch and block scan).
constexpr i64 kScanSingleMax = 65536;
constexpr i64 kScanSingleWide = 16384;
template <typename T, int NT>
constexpr int kScanSingleItems = sizeof(T) == 8 && NT > 256 ? 8 : 16;

template <typename T, int NT>
__global__ void __launch_bounds__(NT) k_scan_single(const T* in, T* out, i64 n_host, const int32_t* d_n,
                                                    T* total_out) {
  __shared__ T s_wave[NT / kWave];
  block_scan_all<T, NT, kScanSingleItems<T, NT>>(in, out, clamp_n(n_host, d_n), total_out, s_wave);
}

template <typename T>
__global__ void __launch_bounds__(kScanThreads) k_scan_reduce(const T* in, T* partial, i64 n_host,
                                                              const int32_t* d_n) {
  __shared__ T s_wave[kScanThreads / kWave];
  const i64 n = clamp_n(n_host, d_n);
  const i64 base = (i64)blockIdx.x * kScanTile + threadIdx.x;
  T sum = 0;
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) {
    const i64 i = base + (i64)k * kScanThreads;
    if (i < n) sum += in[i];
  }
  T total;
  (void)block_excl_scan<T, kScanThreads>(sum, s_wave, total);
  if (threadIdx.x == 0) partial[blockIdx.x] = total;
}

// One workgroup: exclusive scan of the per-block partials, in place, chunk by chunk.
template <typename T>
__global__ void __launch_bounds__(kScanThreads) k_scan_partials(T* partial, i64 nblk, T* out, i64 n_host,
                                                                const int32_t* d_n, T* total_out) {
  __shared__ T s_wave[kScanThreads / kWave];
  T carry = 0;
  for (i64 c = 0; c < nblk; c += kScanTile) {
    T v[kScanItems];
    T sum = 0;
    const i64 base = c + (i64)threadIdx.x * kScanItems;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
      const i64 i = base + k;
      v[k] = i < nblk ? partial[i] : T(0);
      sum += v[k];
    }
    T total;
    T excl = block_excl_scan<T, kScanThreads>(sum, s_wave, total) + carry;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
      const i64 i = base + k;
      if (i < nblk) partial[i] = excl;
      excl += v[k];
    }
    carry += total;
  }
  if (threadIdx.x == 0) {
    out[clamp_n(n_host, d_n)] = carry;
    if (total_out) *total_out = carry;
  }
}

template <typename T>
__global__ void __launch_bounds__(kScanThreads) k_scan_down(const T* in, T* out, const T* partial, i64 n_host,
                                                            const int32_t* d_n) {
  __shared__ T s_tab[kWave + 1];
  const i64 n = clamp_n(n_host, d_n);
  const i64 base = (i64)blockIdx.x * kScanTile + threadIdx.x;
  if ((i64)blockIdx.x * kScanTile >= n) return;  // uniform per block
  T v[kScanItems], ex[kScanItems];
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) {
    const i64 i = base + (i64)k * kScanThreads;
    v[k] = i < n ? in[i] : T(0);
  }
  (void)tile_scan_striped(v, ex, s_tab);
  const T off = partial[blockIdx.x];
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) {
    const i64 i = base + (i64)k * kScanThreads;
    if (i < n) out[i] = ex[k] + off;
  }
}

size_t scan_tmp_bytes(i64 n_host, size_t elem) {
  return n_host <= kScanSingleMax ? 0 : elem * (size_t)ceil_div(n_host, kScanTile);
}

template <typename T>
static void scan_excl(const char* tag, const T* in, T* out, i64 n_host, const int32_t* d_n, hipStream_t s,
                      T* total_out, void* tmp) {
  (void)tag;
  if (n_host <= 0) {
    // n is zero: out[0] = 0
    launch("k_scan_single", k_scan_single<T, 256>, 1, 256, s, in, out, (i64)0, (const int32_t*)nullptr,
           total_out);
    return;
  }
  if (n_host <= kScanSingleWide) {
    launch("k_scan_single", k_scan_single<T, 256>, 1, 256, s, in, out, n_host, d_n, total_out);
    return;
  }
  if (n_host <= kScanSingleMax) {
    launch("k_scan_single", k_scan_single<T, 1024>, 1, 1024, s, in, out, n_host, d_n, total_out);
    return;
  }
  const i64 nblk = ceil_div(n_host, kScanTile);
  Arena a(s);  // used only when the caller brings no scratch
  T* partial = static_cast<T*>(tmp);
  if (!partial) {
    const size_t o = a.reserve(sizeof(T) * (size_t)nblk);
    a.commit();
    partial = a.at<T>(o);
  }
  launch("k_scan_reduce", k_scan_reduce<T>, nblk, kScanThreads, s, in, partial, n_host, d_n);
  launch("k_scan_partials", k_scan_partials<T>, 1, kScanThreads, s, partial, nblk, out, n_host, d_n, total_out);
  launch("k_scan_down", k_scan_down<T>, nblk, kScanThreads, s, in, out, (const T*)partial, n_host, d_n);
}

void scan_excl_i32(const int32_t* in, int32_t* out, i64 n_host, const int32_t* d_n, hipStream_t s,
                   int32_t* total_out, void* tmp) {
  scan_excl("i32", in, out, n_host, d_n, s, total_out, tmp);
}
void scan_excl_i64(const i64* in, i64* out, i64 n_host, const int32_t* d_n, hipStream_t s, i64* total_out,
                   void* tmp) {
  scan_excl("i64", in, out, n_host, d_n, s, total_out, tmp);
}
void scan_excl_u32(const uint32_t* in, uint32_t* out, i64 n_host, const int32_t* d_n, hipStream_t s) {
  scan_excl("u32", in, out, n_host, d_n, s, (uint32_t*)nullptr, nullptr);
}

// ------------------------------------------------------------------ fills
template <typename T>
__global__ void __launch_bounds__(256) k_fill(T* p, T v, i64 n_host, const int32_t* d_n, int32_t mult) {
  i64 n = d_n ? (i64)(*d_n) * mult : n_host;
  if (n > n_host) n = n_host;
  for (i64 i = (i64)blockIdx.x * 256 + threadIdx.x; i < n; i += (i64)gridDim.x * 256) p[i] = v;
}

static i64 fill_blocks(i64 n) {
  i64 b = ceil_div(n, 256);
  return b > 8192 ? 8192 : b;
}

// Two fills in one launch: a[0 .. na) = va and b[0 .. nb) = vb, where na / nb are
// d_n * mult_a / d_n * mult_b when d_n is given (bounded by the host counts).
__global__ void __launch_bounds__(256) k_fill_pair(int32_t* a, int32_t va, i64 na_host, int32_t mult_a, u64* b, u64 vb,
                                                   i64 nb_host, int32_t mult_b, const int32_t* d_n) {
  i64 na = d_n ? (i64)(*d_n) * mult_a : na_host;
  i64 nb = d_n ? (i64)(*d_n) * mult_b : nb_host;
  if (na > na_host) na = na_host;
  if (nb > nb_host) nb = nb_host;
  const i64 stride = (i64)gridDim.x * 256;
  for (i64 i = (i64)blockIdx.x * 256 + threadIdx.x; i < na; i += stride) a[i] = va;
  for (i64 i = (i64)blockIdx.x * 256 + threadIdx.x; i < nb; i += stride) b[i] = vb;
}

void fill_pair(int32_t* a, int32_t va, i64 na_host, int32_t mult_a, u64* b, u64 vb, i64 nb_host, int32_t mult_b,
               const int32_t* d_n, hipStream_t s) {
  launch("k_fill_pair", k_fill_pair, fill_blocks(na_host > nb_host ? na_host : nb_host), 256, s, a, va, na_host,
         mult_a, b, vb, nb_host, mult_b, d_n);
}

void fill_i32(int32_t* p, int32_t v, i64 n_host, const int32_t* d_n, int32_t mult, hipStream_t s) {
  launch("k_fill_i32", k_fill<int32_t>, fill_blocks(n_host), 256, s, p, v, n_host, d_n, mult);
}
void fill_u64(u64* p, u64 v, i64 n_host, const int32_t* d_n, int32_t mult, hipStream_t s) {
  launch("k_fill_u64", k_fill<u64>, fill_blocks(n_host), 256, s, p, v, n_host, d_n, mult);
}

// ------------------------------------------------------------------ sort: bitonic (n <= 4096)
constexpr int kBitonicMax = 4096;
constexpr int kBitonicThreads = 1024;

// (key, value) order: padding entries (all-ones key, value 0xffffffff) stay
// behind every real entry, including real all-ones keys, and equal keys keep
// their value order, so the network is stable.
__device__ __forceinline__ bool key_gt(u64 ahi, u64 alo, uint32_t av, u64 bhi, u64 blo, uint32_t bv) {
  if (ahi != bhi) return ahi > bhi;
  if (alo != blo) return alo > blo;
  return av > bv;
}

__global__ void __launch_bounds__(kBitonicThreads) k_bitonic_sort(Key128* keys, uint32_t* vals, int n, int P) {
  __shared__ u64 s_hi[kBitonicMax];
  __shared__ u64 s_lo[kBitonicMax];
  __shared__ uint32_t s_v[kBitonicMax];
  for (int i = threadIdx.x; i < P; i += kBitonicThreads) {
    if (i < n) {
      const Key128 k = keys[i];
      s_hi[i] = k.hi;
      s_lo[i] = k.lo;
      s_v[i] = vals[i];
    } else {
      s_hi[i] = ~0ull;
      s_lo[i] = ~0ull;
      s_v[i] = 0xffffffffu;
    }
  }
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < P; i += kBitonicThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const bool up = (i & k) == 0;
          const bool gt = key_gt(s_hi[i], s_lo[i], s_v[i], s_hi[ixj], s_lo[ixj], s_v[ixj]);
          const bool lt = key_gt(s_hi[ixj], s_lo[ixj], s_v[ixj], s_hi[i], s_lo[i], s_v[i]);
          if ((up && gt) || (!up && lt)) {
            u64 th = s_hi[i], tl = s_lo[i];
            uint32_t tv = s_v[i];
            s_hi[i] = s_hi[ixj];
            s_lo[i] = s_lo[ixj];
            s_v[i] = s_v[ixj];
            s_hi[ixj] = th;
            s_lo[ixj] = tl;
            s_v[ixj] = tv;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < n; i += kBitonicThreads) {
    keys[i] = Key128{s_lo[i], s_hi[i]};
    vals[i] = s_v[i];
  }
}

// ------------------------------------------------------------------ sort: LSD radix (n > 4096)
constexpr int kRadixThreads = 256;
constexpr int kRadixRounds = 8;
constexpr int kRadixTile = kRadixThreads * kRadixRounds;  // 2048 items per block

__device__ __forceinline__ uint32_t key_digit(const Key128& k, int shift) {
  return shift < 64 ? (uint32_t)((k.lo >> shift) & 255u) : (uint32_t)((k.hi >> (shift - 64)) & 255u);
}

// counts is digit-major: counts[d * nblk + block].
__global__ void __launch_bounds__(kRadixThreads) k_radix_hist(const Key128* keys, i64 n, int shift,
                                                              uint32_t* counts, int nblk) {
  __shared__ uint32_t h[256];
  h[threadIdx.x] = 0;
  __syncthreads();
  const i64 base = (i64)blockIdx.x * kRadixTile;
#pragma unroll
  for (int r = 0; r < kRadixRounds; ++r) {
    const i64 i = base + r * kRadixThreads + threadIdx.x;
    if (i < n) atomicAdd(&h[key_digit(keys[i], shift)], 1u);
  }
  __syncthreads();
  counts[(i64)threadIdx.x * nblk + blockIdx.x] = h[threadIdx.x];
}

// Stable scatter: items are visited in index order (round, wave, lane); ranks
// among equal digits come from wave ballots plus per-wave running counts in LDS.
__global__ void __launch_bounds__(kRadixThreads) k_radix_scatter(const Key128* kin, const uint32_t* vin,
                                                                 Key128* kout, uint32_t* vout, i64 n,
                                                                 int shift, const uint32_t* offs,
                                                                 int nblk) {
  constexpr int kWaves = kRadixThreads / kWave;
  __shared__ uint32_t s_cnt[kWaves][256];
  __shared__ uint32_t s_run[256];
  __shared__ uint32_t s_base[256];
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int lane = tid & (kWave - 1);
  s_run[tid] = 0;
  s_base[tid] = offs[(i64)tid * nblk + blockIdx.x];
#pragma unroll
  for (int q = 0; q < kWaves; ++q) s_cnt[q][tid] = 0;
  __syncthreads();
  const i64 base = (i64)blockIdx.x * kRadixTile;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r = 0; r < kRadixRounds; ++r) {
    const i64 i = base + r * kRadixThreads + tid;
    const bool valid = i < n;
    Key128 key{0, 0};
    uint32_t val = 0;
    uint32_t d = 0;
    if (valid) {
      key = kin[i];
      val = vin[i];
      d = key_digit(key, shift);
    }
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (d >> b) & 1u;
      const uint64_t bb = __ballot(bit);
      peers &= bit ? bb : ~bb;
    }
    const int rank = __popcll(peers & lt_mask);
    if (valid && rank == 0) s_cnt[w][d] = (uint32_t)__popcll(peers);
    __syncthreads();
    {
      const uint32_t run = s_run[tid];
      uint32_t acc = run;
#pragma unroll
      for (int q = 0; q < kWaves; ++q) {
        const uint32_t c = s_cnt[q][tid];
        s_cnt[q][tid] = acc;
        acc += c;
      }
      s_run[tid] = acc;
    }
    __syncthreads();
    if (valid) {
      const uint32_t pos = s_base[d] + s_cnt[w][d] + (uint32_t)rank;
      if ((i64)pos < n) {
        kout[pos] = key;
        vout[pos] = val;
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kWaves; ++q) s_cnt[q][tid] = 0;
    __syncthreads();
  }
}

void sort_pairs_128(Key128* keys, uint32_t* vals, i64 n, int key_bits, hipStream_t s) {
  if (n <= 1) return;
  if (n > 0xffffffffLL) throw Error(TC_ERR_UNSUPPORTED, "sort: too many items");
  if (n <= kBitonicMax) {
    int P = 2;
    while (P < n) P <<= 1;
    launch("k_bitonic_sort", k_bitonic_sort, 1, kBitonicThreads, s, keys, vals, (int)n, P);
    return;
  }
  const int ndig = (key_bits + 7) / 8;
  const i64 nblk = ceil_div(n, kRadixTile);
  if (nblk * 256 > 0x7fffffffLL) throw Error(TC_ERR_UNSUPPORTED, "sort: too many blocks");
  Arena a(s);
  const size_t o_k = a.reserve(sizeof(Key128) * (size_t)n);
  const size_t o_v = a.reserve(sizeof(uint32_t) * (size_t)n);
  const size_t o_c = a.reserve(sizeof(uint32_t) * (size_t)(256 * nblk));
  const size_t o_o = a.reserve(sizeof(uint32_t) * (size_t)(256 * nblk + 1));
  a.commit();
  Key128* kb[2] = {keys, a.at<Key128>(o_k)};
  uint32_t* vb[2] = {vals, a.at<uint32_t>(o_v)};
  uint32_t* counts = a.at<uint32_t>(o_c);
  uint32_t* offs = a.at<uint32_t>(o_o);
  int cur = 0;
  for (int dgt = 0; dgt < ndig; ++dgt) {
    const int shift = dgt * 8;
    launch("k_radix_hist", k_radix_hist, nblk, kRadixThreads, s, (const Key128*)kb[cur], n, shift, counts,
           (int)nblk);
    scan_excl_u32(counts, offs, 256 * nblk, nullptr, s);
    launch("k_radix_scatter", k_radix_scatter, nblk, kRadixThreads, s, (const Key128*)kb[cur],
           (const uint32_t*)vb[cur], kb[cur ^ 1], vb[cur ^ 1], n, shift, (const uint32_t*)offs, (int)nblk);
    cur ^= 1;
  }
  if (cur != 0) {
    hip_check(hipMemcpyAsync(keys, kb[1], sizeof(Key128) * (size_t)n, hipMemcpyDeviceToDevice, s), "sort copy");
    hip_check(hipMemcpyAsync(vals, vb[1], sizeof(uint32_t) * (size_t)n, hipMemcpyDeviceToDevice, s), "sort copy");
  }
}

}  // namespace tc
