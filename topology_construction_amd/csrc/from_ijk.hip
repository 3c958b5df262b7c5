// Grid batch from int32 voxel rows: the ijk emission front-end (PR page,
// Measurements: the follow-up ijk front-end on the same back-end; Test plan:
// expected topologies are built from ijk).
//
// Every voxel emits a single bit. Root tiles are deduplicated with an
// open-addressing hash set (slots hold the index of a representative voxel), the
// few unique tiles are sorted, and the rest reuses the bitmap-rank tree assembly
// of the topology pass. Three small readbacks size the scratch arrays (unique
// tiles, candidate lowers, node counts); the pass itself needs only one because
// its bounds are known from the source batch.
#include <cstring>

#include "device.hpp"
#include "internal.hpp"

namespace tc {

// Member of voxel i: the last g with offsets[g] <= i (binary search).
__device__ __forceinline__ int32_t member_of(const i64* offsets, int32_t B, i64 i) {
  int32_t lo = 0, hi = B - 1;
  while (lo < hi) {
    const int32_t mid = lo + (hi - lo + 1) / 2;
    if (offsets[mid] <= i) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// With at most kLdsMembers members the hashing kernel searches the member
// offsets in LDS.
constexpr int kLdsMembers = 4095;

// Voxels that arrive together usually share their tile, so the lanes of a
// wave that hash the same (grid, tile) probe once, through one leader (up to
// kDedupRounds distinct tiles per wave, found with ballots and shuffles); the
// rest probe on their own.
constexpr int kDedupRounds = 8;


__device__ __forceinline__ u64 wave_or_u64(u64 v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v |= __shfl_xor(v, d, kWave);
  return v;
}

// Ballot merge, for words that most voxels of a wave share (a tile's lower
// bits): the union this lane has to OR into `word` (0 if none) is its group's
// union when it leads a group of lanes with the same word, or its own bits when
// it is left over after kDedupRounds groups.
__device__ __forceinline__ u64 wave_merge_bits(const u64* word, u64 bits, bool active) {
  const int lane = threadIdx.x & (kWave - 1);
  u64 todo = __ballot(active);
  u64 mine = 0;
  for (int round = 0; todo && round < kDedupRounds; ++round) {
    const int leader = __builtin_ctzll(todo);
    const u64 lw = (u64)__shfl((long long)(uintptr_t)word, leader, kWave);
    const bool same = ((todo >> lane) & 1ull) && (u64)(uintptr_t)word == lw;
    const u64 sm = __ballot(same);
    const u64 all = wave_or_u64(same ? bits : 0);
    if (lane == leader) mine = all;
    todo &= ~sm;
  }
  if ((todo >> lane) & 1ull) mine = bits;
  return mine;
}

// Candidate and leaf words are many (about ten leaf words per 64 consecutive
// voxels of a shell, ~95 per 1024): there the block ORs the bits of its
// kVoxPerBlock voxels into an LDS hash table keyed by word address (LDS
// compare-and-swap claims a key, LDS OR merges the bits), then ORs each
// distinct word once, all of them at once. With kCheck the global word is read
// first and the OR skipped when its bits are already set.
constexpr int kBlockTable = 2048;  // entries; at most kVoxPerBlock keys, so probes stay short

__device__ __forceinline__ void table_clear(unsigned long long* key, unsigned long long* val) {
  for (int e = threadIdx.x; e < kBlockTable; e += 256) {
    key[e] = 0ull;
    val[e] = 0ull;
  }
}

// Every insert finds its key or a free entry within kBlockTable probes because
// the table holds at most kVoxPerBlock keys.
__device__ __forceinline__ void table_or(unsigned long long* key, unsigned long long* val, const u64* word, u64 bits) {
  const unsigned long long k = (unsigned long long)(uintptr_t)word;
  unsigned h = (unsigned)(((k >> 3) * 0x9e3779b97f4a7c15ull) >> 53);  // 11 bits
  for (int probe = 0; probe < kBlockTable; ++probe) {
    const unsigned long long prev = atomicCAS(&key[h], 0ull, k);
    if (prev == 0ull || prev == k) {
      atomicOr(&val[h], (unsigned long long)bits);
      return;
    }
    h = (h + 1) & (kBlockTable - 1);
  }
}

template <bool kCheck>
__device__ __forceinline__ void table_flush(const unsigned long long* key, const unsigned long long* val) {
  constexpr int kPer = kBlockTable / 256;
  unsigned long long k[kPer], v[kPer], cur[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    k[j] = key[threadIdx.x + 256 * j];
    v[j] = val[threadIdx.x + 256 * j];
  }
  if (kCheck) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) cur[j] = k[j] ? *reinterpret_cast<const u64*>((uintptr_t)k[j]) : 0ull;
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (k[j] && (!kCheck || (cur[j] & v[j]) != v[j]))
      atomicOr(reinterpret_cast<unsigned long long*>((uintptr_t)k[j]), v[j]);
}

// Voxels per lane of the per-voxel kernels: slot v of a wave covers the 64
// consecutive voxels base + 64 v + lane, and the slots' loads go out together.
// The kernels that merge through the block's LDS table take kVoxPerLane voxels
// per lane (the table holds twice the block's voxels); the others take
// kVoxPerLaneWide (more loads in flight per wave).
constexpr int kVoxPerLane = 4;
constexpr int kVoxPerBlock = 256 * kVoxPerLane;
constexpr int kVoxPerLaneWide = 8;
constexpr int kVoxPerBlockWide = 256 * kVoxPerLaneWide;

template <int V>
__device__ __forceinline__ i64 vox_index(int v) {
  return (i64)blockIdx.x * (256 * V) + (threadIdx.x / kWave) * (kWave * V) + v * kWave + (threadIdx.x & (kWave - 1));
}

__device__ __forceinline__ u64 tile_hash(int32_t g, int32_t tx, int32_t ty, int32_t tz) {
  u64 k = ((u64)(uint32_t)(tx + kTileBias) << 40) ^ ((u64)(uint32_t)(ty + kTileBias) << 20) ^
          (u64)(uint32_t)(tz + kTileBias);
  k ^= (u64)(uint32_t)g * 0x9e3779b97f4a7c15ull;
  k ^= k >> 31;
  k *= 0xbf58476d1ce4e5b9ull;
  k ^= k >> 29;
  k *= 0x94d049bb133111ebull;
  k ^= k >> 32;
  return k;
}

// table[H] holds -1 or the index of the first voxel seen for a (grid, tile).
// Every probe sequence ends within H steps because fewer than H voxels exist.
// Returns the representative voxel of voxel i's (grid, tile).
__device__ int32_t tile_probe(const int32_t* ijk, const i64* offsets, int32_t B, i64 i, int32_t g, int32_t tx,
                              int32_t ty, int32_t tz, int32_t* table, i64 H, int32_t* flags) {
  i64 h = (i64)(tile_hash(g, tx, ty, tz) & (u64)(H - 1));
  for (i64 probe = 0; probe < H; ++probe) {
    int32_t e = __hip_atomic_load(&table[h], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (e < 0) {
      const int32_t old = atomicCAS(&table[h], -1, (int32_t)i);
      if (old < 0) return (int32_t)i;
      e = old;
    }
    if ((ijk[(i64)e * 3] >> 12) == tx && (ijk[(i64)e * 3 + 1] >> 12) == ty && (ijk[(i64)e * 3 + 2] >> 12) == tz &&
        member_of(offsets, B, e) == g)
      return e;
    h = (h + 1) & (H - 1);
  }
  atomicOr(flags, 2);
  return (int32_t)i;
}

// Lanes of a wave that share a (grid, tile) probe once, through one leader, and
// a key equal to the wave's previous one reuses its result without probing
// (voxels that arrive together share their tile, so one probe per wave is
// typical). kVoxPerLaneWide voxels per lane (slots), their loads and member
// searches together. Also flags the representatives (rep[i] == i): exactly the
// voxels whose probe inserted their own index.
__global__ void __launch_bounds__(256) k_hash_tiles(const int32_t* ijk, const i64* offsets, int32_t B, i64 n,
                                                    int32_t* table, i64 H, int32_t* rep, int32_t* is_rep,
                                                    int32_t* flags) {
  constexpr int V = kVoxPerLaneWide;
  __shared__ i64 s_off[kLdsMembers + 1];
  const bool lds = B <= kLdsMembers;  // uniform
  const int lane = threadIdx.x & (kWave - 1);
  bool in[V];
  int32_t tx[V], ty[V], tz[V], g[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const i64 i = vox_index<V>(v);
    in[v] = i < n;
    tx[v] = in[v] ? ijk[i * 3] >> 12 : 0;
    ty[v] = in[v] ? ijk[i * 3 + 1] >> 12 : 0;
    tz[v] = in[v] ? ijk[i * 3 + 2] >> 12 : 0;
  }
  if (lds) {
    for (int k = threadIdx.x; k <= B; k += 256) s_off[k] = offsets[k];
    __syncthreads();
  }
  const i64* off = lds ? s_off : offsets;
#pragma unroll
  for (int v = 0; v < V; ++v) g[v] = in[v] ? member_of(off, B, vox_index<V>(v)) : 0;
  // the wave's last resolved key and its representative (uniform)
  int32_t kg = -1, kx = 0, ky = 0, kz = 0, krep = -1;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const i64 i = vox_index<V>(v);
    int32_t mine = -1;
    u64 todo = __ballot(in[v]);
    for (int round = 0; todo && round < kDedupRounds; ++round) {
      const int leader = __builtin_ctzll(todo);
      const int32_t lg = __shfl(g[v], leader, kWave), lx = __shfl(tx[v], leader, kWave),
                    ly = __shfl(ty[v], leader, kWave), lz = __shfl(tz[v], leader, kWave);
      const bool same = ((todo >> lane) & 1ull) && g[v] == lg && tx[v] == lx && ty[v] == ly && tz[v] == lz;
      const u64 sm = __ballot(same);
      int32_t r;
      if (lg == kg && lx == kx && ly == ky && lz == kz) {
        r = krep;
      } else {
        r = -1;
        if (lane == leader) r = tile_probe(ijk, off, B, i, lg, lx, ly, lz, table, H, flags);
        r = __shfl(r, leader, kWave);
        kg = lg;
        kx = lx;
        ky = ly;
        kz = lz;
        krep = r;
      }
      if (same) mine = r;
      todo &= ~sm;
    }
    if ((todo >> lane) & 1ull) mine = tile_probe(ijk, off, B, i, g[v], tx[v], ty[v], tz[v], table, H, flags);
    if (in[v]) {
      rep[i] = mine;
      is_rep[i] = mine == i ? 1 : 0;
    }
  }
}

__global__ void __launch_bounds__(256) k_tile_compact(const int32_t* ijk, const i64* offsets, int32_t B,
                                                      const int32_t* flag, const int32_t* excl, i64 n, Key128* keys,
                                                      uint32_t* vals) {
  const i64 i = (i64)blockIdx.x * 256 + threadIdx.x;
  if (i >= n || !flag[i]) return;
  const int32_t k = excl[i];
  const u64 g = (uint32_t)member_of(offsets, B, i);
  const u64 tx = (u64)((ijk[i * 3] >> 12) + kTileBias), ty = (u64)((ijk[i * 3 + 1] >> 12) + kTileBias),
            tz = (u64)((ijk[i * 3 + 2] >> 12) + kTileBias);
  keys[k] = Key128{((g & 15ull) << 60) | (tx << 40) | (ty << 20) | tz, g >> 4};
  vals[k] = (uint32_t)k;
}

__global__ void __launch_bounds__(256) k_tile_rank_scatter(const Key128* keys, const uint32_t* vals, i64 n,
                                                           int32_t* rank_of, int4* utile) {
  const i64 s = (i64)blockIdx.x * 256 + threadIdx.x;
  if (s >= n) return;
  const Key128 k = keys[s];
  if ((i64)vals[s] >= n) return;  // consistency guard
  rank_of[vals[s]] = (int32_t)s;
  const int32_t g = (int32_t)((k.hi << 4) | (k.lo >> 60));
  utile[s] = make_int4((int32_t)((k.lo >> 40) & 0xfffff) - kTileBias, (int32_t)((k.lo >> 20) & 0xfffff) - kTileBias,
                       (int32_t)(k.lo & 0xfffff) - kTileBias, g);
}

__global__ void __launch_bounds__(256) k_voxel_tile(const int32_t* rep, const int32_t* excl, const int32_t* rank_of,
                                                    i64 n, int32_t nt, int32_t* vtile, int32_t* flags) {
  constexpr int V = kVoxPerLaneWide;
  int32_t r[V], k[V], t[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const i64 i = vox_index<V>(v);
    r[v] = i < n ? rep[i] : -1;
  }
#pragma unroll
  for (int v = 0; v < V; ++v) k[v] = (r[v] >= 0 && r[v] < n) ? excl[r[v]] : -1;
#pragma unroll
  for (int v = 0; v < V; ++v) t[v] = (k[v] >= 0 && k[v] < nt) ? rank_of[k[v]] : -1;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const i64 i = vox_index<V>(v);
    if (i >= n) continue;
    if (t[v] < 0 || t[v] >= nt) {
      atomicOr(flags, 2);
      vtile[i] = 0;
    } else {
      vtile[i] = t[v];
    }
  }
}

__global__ void __launch_bounds__(256) k_voxel_mark_lower(const int32_t* ijk, const int32_t* vtile, i64 n,
                                                          u64* tile_child) {
  constexpr int V = kVoxPerLaneWide;
  u64* word[V];
  u64 b[V];
  bool in[V];
  int32_t t[V], x[V], y[V], z[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const i64 i = vox_index<V>(v);
    in[v] = i < n;
    t[v] = in[v] ? vtile[i] : 0;
    x[v] = in[v] ? ijk[i * 3] : 0;
    y[v] = in[v] ? ijk[i * 3 + 1] : 0;
    z[v] = in[v] ? ijk[i * 3 + 2] : 0;
  }
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int bit = ((((x[v] >> 7) & 31) * 32 + ((y[v] >> 7) & 31)) * 32) + ((z[v] >> 7) & 31);
    word[v] = in[v] ? &tile_child[(i64)t[v] * 512 + (bit >> 6)] : tile_child;
    b[v] = in[v] ? 1ull << (bit & 63) : 0ull;
  }
  u64 mine[V], cur[V];
#pragma unroll
  for (int v = 0; v < V; ++v) mine[v] = wave_merge_bits(word[v], b[v], in[v]);
#pragma unroll
  for (int v = 0; v < V; ++v) cur[v] = mine[v] ? *word[v] : 0ull;  // the reads go out together
#pragma unroll
  for (int v = 0; v < V; ++v)
    if (mine[v] && (cur[v] & mine[v]) != mine[v]) atomicOr((unsigned long long*)word[v], mine[v]);
}

// All lanes stay active to the end of these kernels (no early return), so the
// wave-wide merges see every lane.
__global__ void __launch_bounds__(256) k_voxel_cand(const int32_t* ijk, const int32_t* vtile, i64 n,
                                                    const u64* tile_child, const uint16_t* tile_prefix,
                                                    const int32_t* tile_lower_base, int32_t nc, int32_t* vcand,
                                                    int4* cand_origin, u64* cand_child, int32_t* flags) {
  constexpr int V = kVoxPerLane;
  __shared__ unsigned long long s_key[kBlockTable], s_val[kBlockTable];
  table_clear(s_key, s_val);
  const int lane = threadIdx.x & (kWave - 1);
  bool ok[V];
  int32_t t[V], x[V], y[V], z[V], c[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const i64 i = vox_index<V>(v);
    ok[v] = i < n;
    t[v] = ok[v] ? vtile[i] : 0;
    x[v] = ok[v] ? ijk[i * 3] : 0;
    y[v] = ok[v] ? ijk[i * 3 + 1] : 0;
    z[v] = ok[v] ? ijk[i * 3 + 2] : 0;
  }
  int w[V], bb[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int bit = (((x[v] >> 7) & 31) * 32 + ((y[v] >> 7) & 31)) * 32 + ((z[v] >> 7) & 31);
    w[v] = bit >> 6;
    bb[v] = bit & 63;
  }
  int32_t base[V];
  uint16_t pre[V];
  u64 cw[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const i64 tt = ok[v] ? t[v] : 0;
    base[v] = tile_lower_base[tt];
    pre[v] = tile_prefix[tt * 512 + w[v]];
    cw[v] = tile_child[tt * 512 + w[v]];
  }
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const i64 i = vox_index<V>(v);
    c[v] = -1;
    if (ok[v]) {
      c[v] = base[v] + pre[v] + popc64(cw[v] & ((1ull << bb[v]) - 1));
      if (c[v] < 0 || c[v] >= nc) {
        atomicOr(flags, 2);
        c[v] = -1;
        ok[v] = false;
      }
      vcand[i] = c[v];
    }
  }
  // one lane per run of equal candidates writes the candidate's origin
  u64* word[V];
  u64 bits[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int32_t cprev = __shfl_up(c[v], 1, kWave);
    if (ok[v] && (lane == 0 || cprev != c[v]))
      cand_origin[c[v]] = make_int4((x[v] >> 7) * 128, (y[v] >> 7) * 128, (z[v] >> 7) * 128, t[v]);
    const int lb = (((x[v] >> 3) & 15) * 16 + ((y[v] >> 3) & 15)) * 16 + ((z[v] >> 3) & 15);
    word[v] = ok[v] ? &cand_child[(i64)c[v] * 64 + (lb >> 6)] : cand_child;
    bits[v] = ok[v] ? 1ull << (lb & 63) : 0ull;
  }
  __syncthreads();  // the cleared table
#pragma unroll
  for (int v = 0; v < V; ++v)
    if (ok[v]) table_or(s_key, s_val, word[v], bits[v]);
  __syncthreads();
  table_flush<true>(s_key, s_val);
}

__global__ void __launch_bounds__(256) k_voxel_leaf(const int32_t* ijk, const int32_t* vcand, i64 n,
                                                    const u64* cand_child, const uint16_t* cand_prefix,
                                                    const i64* cand_scan, i64 n_leaf, u64* leaf_mask,
                                                    int32_t* flags) {
  constexpr int V = kVoxPerLane;
  __shared__ unsigned long long s_key[kBlockTable], s_val[kBlockTable];
  table_clear(s_key, s_val);
  bool ok[V];
  int32_t c[V], x[V], y[V], z[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const i64 i = vox_index<V>(v);
    const bool in = i < n;
    c[v] = in ? vcand[i] : -1;
    x[v] = in ? ijk[i * 3] : 0;
    y[v] = in ? ijk[i * 3 + 1] : 0;
    z[v] = in ? ijk[i * 3 + 2] : 0;
    ok[v] = in && c[v] >= 0;
  }
  bool bad = false;
#pragma unroll
  for (int v = 0; v < V; ++v) bad |= (vox_index<V>(v) < n) && !ok[v];  // every voxel has its candidate lower
  int w[V], b[V];
  i64 sc[V];
  uint16_t pre[V];
  u64 cw[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int lb = (((x[v] >> 3) & 15) * 16 + ((y[v] >> 3) & 15)) * 16 + ((z[v] >> 3) & 15);
    w[v] = lb >> 6;
    b[v] = lb & 63;
    const i64 cc = ok[v] ? c[v] : 0;
    sc[v] = cand_scan[cc];
    pre[v] = cand_prefix[cc * 64 + w[v]];
    cw[v] = cand_child[cc * 64 + w[v]];
  }
  u64* word[V];
  u64 bits[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    word[v] = leaf_mask;
    bits[v] = 0;
    if (ok[v]) {
      const i64 leaf = (i64)(sc[v] & 0xffffffffll) + pre[v] + popc64(cw[v] & ((1ull << b[v]) - 1));
      if (leaf < 0 || leaf >= n_leaf) {  // consistency guard
        ok[v] = false;
        bad = true;
      } else {
        word[v] = &leaf_mask[leaf * 8 + (x[v] & 7)];
        bits[v] = 1ull << ((y[v] & 7) * 8 + (z[v] & 7));
      }
    }
  }
  __syncthreads();  // the cleared table
  if (bad) atomicOr(flags, 2);
#pragma unroll
  for (int v = 0; v < V; ++v)
    if (ok[v]) table_or(s_key, s_val, word[v], bits[v]);
  __syncthreads();
  table_flush<false>(s_key, s_val);
}

// Two device words read back with one synchronisation. The pinned staging
// buffer may still be the source of an earlier upload on the stream: the
// copies into it are ordered after that upload by the stream itself.
static void read_two_i32(const int32_t* d0, const int32_t* d1, hipStream_t s, int32_t* v0, int32_t* v1) {
  int32_t* h = static_cast<int32_t*>(pinned_staging(64));
  hip_check(hipMemcpyAsync(h, d0, 4, hipMemcpyDeviceToHost, s), "readback");
  hip_check(hipMemcpyAsync(h + 1, d1, 4, hipMemcpyDeviceToHost, s), "readback");
  hip_check(hipStreamSynchronize(s), "hipStreamSynchronize");
  *v0 = h[0];
  *v1 = h[1];
}

tc_grid_batch* build_from_ijk(const int32_t* d_ijk, const int64_t* h_off, int32_t B, const OutAlloc& oa) {
  hipStream_t s = oa.stream;
  const i64 N = h_off[B];
  i64 H = 1024;
  while (H < 2 * N) H <<= 1;

  // stage 1: voxel -> grid, tile representatives, unique tiles
  Arena a1(s);
  const size_t o_off = a1.reserve(8 * ((i64)B + 1));
  const size_t o_tab = a1.reserve(4 * H);
  const size_t o_rep = a1.reserve(4 * N);
  const size_t o_flag = a1.reserve(4 * N);
  const size_t o_excl = a1.reserve(4 * (N + 1));
  const size_t o_vt = a1.reserve(4 * N);
  const size_t o_vc = a1.reserve(4 * N);
  const size_t o_rb = a1.reserve(4 * 4);
  a1.commit();
  i64* d_off = a1.at<i64>(o_off);
  int32_t* table = a1.at<int32_t>(o_tab);
  int32_t* rep = a1.at<int32_t>(o_rep);
  int32_t* flag = a1.at<int32_t>(o_flag);
  int32_t* excl = a1.at<int32_t>(o_excl);
  int32_t* vtile = a1.at<int32_t>(o_vt);
  int32_t* vcand = a1.at<int32_t>(o_vc);
  int32_t* flags = a1.at<int32_t>(o_rb);

  const size_t off_bytes = 8 * ((size_t)B + 1);
  void* h_stage = pinned_staging(off_bytes + 64);
  std::memcpy(h_stage, h_off, off_bytes);
  hip_check(hipMemcpyAsync(d_off, h_stage, off_bytes, hipMemcpyHostToDevice, s), "offsets upload");
  fill_i32(flags, 0, 1, nullptr, 1, s);
  fill_i32(table, -1, H, nullptr, 1, s);
  launch("k_hash_tiles", k_hash_tiles, ceil_div(N, kVoxPerBlockWide), 256, s, d_ijk, (const i64*)d_off, B, N, table, H,
         rep, flag, flags);
  scan_excl_i32(flag, excl, N, nullptr, s);
  int32_t nt = 0, hash_flags = 0;
  read_two_i32(excl + N, flags, s, &nt, &hash_flags);
  if (hash_flags & 2) throw Error(TC_ERR_INTERNAL, "from_ijk: tile hash overflow");

  // stage 2: sort the unique tiles, candidate lowers
  Arena a2(s);
  const size_t o_keys = a2.reserve(sizeof(Key128) * nt);
  const size_t o_vals = a2.reserve(4 * (i64)nt);
  const size_t o_rank = a2.reserve(4 * (i64)nt);
  const size_t o_ntiles = a2.reserve(4);
  const size_t o_ncand = a2.reserve(4);
  const size_t o_utile = a2.reserve(16 * (i64)nt);
  const size_t o_tchild = a2.reserve(4096 * (i64)nt);
  const size_t o_tpre = a2.reserve(1024 * (i64)nt);
  const size_t o_tlc = a2.reserve(4 * (i64)nt);
  const size_t o_tlb = a2.reserve(4 * ((i64)nt + 1));
  const size_t o_tne = a2.reserve(4 * (i64)nt);
  const size_t o_uex = a2.reserve(4 * ((i64)nt + 1));
  const size_t o_gtb = a2.reserve(4 * ((i64)B + 1));
  a2.commit();
  TreeScratch ts{};
  ts.cap_tiles = nt;
  ts.d_num_tiles = a2.at<int32_t>(o_ntiles);
  ts.d_num_cands = a2.at<int32_t>(o_ncand);
  ts.utile = a2.at<int4>(o_utile);
  ts.tile_child = a2.at<u64>(o_tchild);
  ts.tile_prefix = a2.at<uint16_t>(o_tpre);
  ts.tile_lower_count = a2.at<int32_t>(o_tlc);
  ts.tile_lower_base = a2.at<int32_t>(o_tlb);
  ts.tile_nonempty = a2.at<int32_t>(o_tne);
  ts.upper_excl = a2.at<int32_t>(o_uex);
  ts.grid_tile_begin = a2.at<int32_t>(o_gtb);
  Key128* keys = a2.at<Key128>(o_keys);
  uint32_t* vals = a2.at<uint32_t>(o_vals);
  int32_t* rank_of = a2.at<int32_t>(o_rank);

  fill_i32(ts.d_num_tiles, nt, 1, nullptr, 1, s);
  launch("k_tile_compact", k_tile_compact, ceil_div(N, 256), 256, s, d_ijk, (const i64*)d_off, B,
         (const int32_t*)flag, (const int32_t*)excl, N, keys, vals);
  sort_pairs_128(keys, vals, nt, tile_key_bits(B), s);
  launch("k_tile_rank_scatter", k_tile_rank_scatter, ceil_div(nt, 256), 256, s, (const Key128*)keys,
         (const uint32_t*)vals, (i64)nt, rank_of, ts.utile);
  launch("k_voxel_tile", k_voxel_tile, ceil_div(N, kVoxPerBlockWide), 256, s, (const int32_t*)rep, (const int32_t*)excl,
         (const int32_t*)rank_of, N, nt, vtile, flags);
  tree_tile_ranges(ts, B, s);
  fill_u64(ts.tile_child, 0, 512 * (i64)nt, nullptr, 1, s);
  launch("k_voxel_mark_lower", k_voxel_mark_lower, ceil_div(N, kVoxPerBlockWide), 256, s, d_ijk, (const int32_t*)vtile, N,
         ts.tile_child);
  tree_rank_tiles(ts, s);
  int32_t nc = 0, rank_flags = 0;
  read_two_i32(ts.d_num_cands, flags, s, &nc, &rank_flags);
  if (rank_flags & 2) throw Error(TC_ERR_INTERNAL, "from_ijk: tile ranking check failed");

  // stage 3: candidate lowers, leaves, counts
  Arena a3(s);
  const size_t o_corig = a3.reserve(16 * (i64)nc);
  const size_t o_cchild = a3.reserve(512 * (i64)nc);
  const size_t o_cpre = a3.reserve(128 * (i64)nc);
  const size_t o_clc = a3.reserve(8 * (i64)nc);
  const size_t o_lb = a3.reserve(8 * ((i64)nc + 1));
  const size_t o_ginfo = a3.reserve(4 * 6 * (i64)B);
  const size_t o_rb3 = a3.reserve(4 * (4 + 3 * (i64)B));
  const size_t o_stmp3 = a3.reserve(std::max(scan_tmp_bytes(nt, 4), scan_tmp_bytes(nc, 8)));
  a3.commit();
  ts.cap_cands = nc;
  ts.cand_origin = a3.at<int4>(o_corig);
  ts.cand_child = a3.at<u64>(o_cchild);
  ts.cand_prefix = a3.at<uint16_t>(o_cpre);
  ts.cand_counts = a3.at<i64>(o_clc);
  ts.cand_scan = a3.at<i64>(o_lb);
  ts.grid_info = a3.at<int32_t>(o_ginfo);
  ts.readback = a3.at<int32_t>(o_rb3);
  ts.scan_tmp = a3.at<char>(o_stmp3);
  ts.flags = ts.readback;
  fill_i32(ts.readback, 0, 1, nullptr, 1, s);
  fill_u64(ts.cand_child, 0, 64 * (i64)nc, nullptr, 1, s);
  launch("k_voxel_cand", k_voxel_cand, ceil_div(N, kVoxPerBlock), 256, s, d_ijk, (const int32_t*)vtile, N,
         (const u64*)ts.tile_child, (const uint16_t*)ts.tile_prefix, (const int32_t*)ts.tile_lower_base, nc, vcand,
         ts.cand_origin, ts.cand_child, ts.flags);
  tree_counts(ts, B, s);
  const size_t rb_bytes = 4 * (4 + 3 * (size_t)B);
  int32_t* h_rb = static_cast<int32_t*>(pinned_staging(rb_bytes));
  hip_check(hipMemcpyAsync(h_rb, ts.readback, rb_bytes, hipMemcpyDeviceToHost, s), "readback");
  hip_check(hipStreamSynchronize(s), "hipStreamSynchronize");
  if (h_rb[0] != 0) throw Error(TC_ERR_INTERNAL, "from_ijk: device consistency check failed");

  tc_grid_batch* out = new_batch(B, h_rb, oa);
  try {
    const GridView ov = out->view();
    const i64 L = out->nl;
    Arena post(s);
    const size_t o_lc = post.reserve(4 * L);
    const size_t o_box = post.reserve(4 * L);
    const size_t o_bb = post.reserve(4 * 6 * (i64)B * bbox_replicas(B));
    const size_t o_part = post.reserve(8 * (ceil_div(L, 256) + 1));  // voxel sums per 256 leaves
    const size_t o_gvb = post.reserve(8 * ((i64)B + 1));
    const size_t o_inrun = post.reserve(4 * L);
    post.commit();
    tree_write_nodes(ts, ov, post.at<int32_t>(o_lc), s);
    fill_u64(ov.leaf_mask, 0, 8 * L, nullptr, 1, s);
    launch("k_voxel_leaf", k_voxel_leaf, ceil_div(N, kVoxPerBlock), 256, s, d_ijk, (const int32_t*)vcand, N,
           (const u64*)ts.cand_child, (const uint16_t*)ts.cand_prefix, (const i64*)ts.cand_scan, L,
           ov.leaf_mask, ts.flags);
    tree_leaf_stats(ov, post.at<uint32_t>(o_box), post.at<int32_t>(o_inrun), post.at<i64>(o_part), s);
    apply_debug_inject(ts.flags, s);  // k_voxel_leaf's checks ran after the readback: finalize copies the word
    tree_finalize_leaves(ov, post.at<uint32_t>(o_box), post.at<int32_t>(o_inrun), post.at<i64>(o_part), 256,
                         post.at<i64>(o_gvb), post.at<int32_t>(o_bb), (const int32_t*)ts.grid_info, ts.flags,
                         ts.readback + 3, s);
  } catch (...) {
    free_batch(out);
    throw;
  }
  return out;
}

}  // namespace tc
