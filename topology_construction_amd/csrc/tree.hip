// Tree assembly shared by the topology pass and the ijk front-end.
//
// Input state (TreeScratch): the unique root tiles of the output in canonical
// order (sorted by grid, then signed x-major tile coordinate), for every tile a
// 32^3-bit mask of candidate lower nodes, and for every candidate lower node a
// 16^3-bit mask of its non-empty leaves. Candidate lower nodes are numbered tile
// by tile in mask-bit order, which is the x-major upper-child order, so the
// numbering is already canonical; leaves inside a lower are likewise numbered in
// mask-bit (x-major lower-child) order. Empty candidates are compacted away.
//
// This replaces the per-slot sort and head-flag dedup of the PR page (section 1)
// at leaf level with bitmap marking plus popcount ranks: duplicates collapse in
// the bitmaps and ranks come from prefix popcounts, so no leaf-level sort runs.
#include <algorithm>

#include "device.hpp"
#include "internal.hpp"

namespace tc {

// ------------------------------------------------------------------ tiles
// grid_tile_begin[g] = first unique tile of grid g; grid_tile_begin[B] = num tiles.
__global__ void __launch_bounds__(256) k_grid_tile_ranges(const int4* utile, const int32_t* d_num_tiles,
                                                          int32_t B, int32_t* begin) {
  const i64 t = (i64)blockIdx.x * 256 + threadIdx.x;
  const int32_t nt = *d_num_tiles;
  if (nt == 0) {
    if (t == 0)
      for (int32_t g = 0; g <= B; ++g) begin[g] = 0;
    return;
  }
  if (t >= nt) return;
  const int32_t g = utile[t].w;
  const int32_t gp = t == 0 ? -1 : utile[t - 1].w;
  for (int32_t q = gp + 1; q <= g; ++q) begin[q] = (int32_t)t;
  if (t == nt - 1)
    for (int32_t q = g + 1; q <= B; ++q) begin[q] = nt;
}

void tree_tile_ranges(TreeScratch& ts, int32_t B, hipStream_t s) {
  const i64 n = ts.cap_tiles > 0 ? ts.cap_tiles : 1;
  launch("k_grid_tile_ranges", k_grid_tile_ranges, ceil_div(n, 256), 256, s, (const int4*)ts.utile,
         (const int32_t*)ts.d_num_tiles, B, ts.grid_tile_begin);
}

// One workgroup per tile: per-word exclusive popcount prefix of the 512-word
// candidate-lower mask and the tile's candidate count.
__global__ void __launch_bounds__(256) k_tile_rank(const u64* tile_child, uint16_t* tile_prefix,
                                                   int32_t* tile_lower_count, const int32_t* d_num_tiles) {
  __shared__ int32_t s_wave[4];
  const i64 t = blockIdx.x;
  if (t >= *d_num_tiles) return;
  const int w0 = threadIdx.x * 2;
  const u64 a = tile_child[t * 512 + w0];
  const u64 b = tile_child[t * 512 + w0 + 1];
  const int ca = popc64(a), cb = popc64(b);
  int32_t total;
  const int32_t ex = block_excl_scan<int32_t, 256>(ca + cb, s_wave, total);
  tile_prefix[t * 512 + w0] = (uint16_t)ex;
  tile_prefix[t * 512 + w0 + 1] = (uint16_t)(ex + ca);
  if (threadIdx.x == 0) tile_lower_count[t] = total;
}

// At most kRankLastTiles tiles: k_tile_rank, the scan of the tiles' lower counts
// and the start of the candidate -> source table in one launch. Each tile's
// workgroup writes its prefix table and count, publishes them (device fence)
// and counts itself in done_ctr (zeroed by the tile stage); the last one reads
// every count with device-scope loads, scans them into the tile bases and the
// candidate count, and sets the table's first nc * m_src entries to -1.
constexpr int kRankLastTiles = 4096;

__global__ void __launch_bounds__(256) k_tile_rank_last(const u64* tile_child, uint16_t* tile_prefix,
                                                        int32_t* tile_lower_count, int32_t* tile_lower_base,
                                                        const int32_t* d_num_tiles, int32_t* d_num_cands,
                                                        int32_t* done_ctr, int32_t* cand_src, int32_t m_src) {
  __shared__ int32_t s_wave[4];
  __shared__ int32_t s_last;
  const int32_t nt = *d_num_tiles;
  const i64 t = blockIdx.x;
  const int tid = threadIdx.x;
  if (nt <= 0) {  // no tiles: no workgroup counts itself
    if (t == 0 && tid == 0) {
      tile_lower_base[0] = 0;
      *d_num_cands = 0;
    }
    return;
  }
  if (t >= nt) return;  // uniform per block
  const int w0 = tid * 2;
  const u64 a = tile_child[t * 512 + w0];
  const u64 b = tile_child[t * 512 + w0 + 1];
  const int ca = popc64(a), cb = popc64(b);
  int32_t total;
  const int32_t ex = block_excl_scan<int32_t, 256>(ca + cb, s_wave, total);
  tile_prefix[t * 512 + w0] = (uint16_t)ex;
  tile_prefix[t * 512 + w0 + 1] = (uint16_t)(ex + ca);
  if (tid == 0) {
    tile_lower_count[t] = total;
    __threadfence();
    s_last = atomicAdd(done_ctr, 1) == nt - 1 ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;  // uniform per block
  __threadfence();
  constexpr int kPer = kRankLastTiles / 256;
  int32_t v[kPer];
  int32_t sum = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int i = tid * kPer + k;
    v[k] = i < nt ? __hip_atomic_load(&tile_lower_count[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
    sum += v[k];
  }
  int32_t nc;
  int32_t base = block_excl_scan<int32_t, 256>(sum, s_wave, nc);
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int i = tid * kPer + k;
    if (i < nt) tile_lower_base[i] = base;
    base += v[k];
  }
  if (tid == 0) {
    tile_lower_base[nt] = nc;
    *d_num_cands = nc;
  }
  for (i64 e = tid; e < (i64)nc * m_src; e += 256) cand_src[e] = -1;
}

void tree_rank_tiles_last(TreeScratch& ts, int32_t* done_ctr, int32_t* cand_src, int32_t m_src, hipStream_t s) {
  if (ts.cap_tiles > kRankLastTiles) throw Error(TC_ERR_INTERNAL, "rank: too many tiles for the one-launch stage");
  launch("k_tile_rank", k_tile_rank_last, std::max<i64>(1, ts.cap_tiles), 256, s, (const u64*)ts.tile_child,
         ts.tile_prefix, ts.tile_lower_count, ts.tile_lower_base, (const int32_t*)ts.d_num_tiles, ts.d_num_cands,
         done_ctr, cand_src, m_src);
}

void tree_rank_tiles(TreeScratch& ts, hipStream_t s) {
  launch("k_tile_rank", k_tile_rank, ts.cap_tiles, 256, s, (const u64*)ts.tile_child, ts.tile_prefix,
         ts.tile_lower_count, (const int32_t*)ts.d_num_tiles);
  // the total of the scan is the number of candidate lowers
  scan_excl_i32(ts.tile_lower_count, ts.tile_lower_base, ts.cap_tiles, ts.d_num_tiles, s, ts.d_num_cands,
                ts.scan_tmp);
}

// ------------------------------------------------------------------ candidate lowers
// cand_counts[c] packs the candidate's leaf count (low 32 bits) and its
// non-empty flag (high 32 bits); one 64-bit exclusive scan then gives, per
// candidate, its first output leaf (low half) and its output lower index (high
// half). Totals stay below 2^31, so the halves never carry into each other.
__device__ __forceinline__ int32_t scan_leaf(i64 v) { return (int32_t)(v & 0xffffffffll); }
__device__ __forceinline__ int32_t scan_lower(i64 v) { return (int32_t)(v >> 32); }

// One wave per candidate lower: per-word exclusive popcount prefix of its 64-word
// leaf mask and its packed count.
__global__ void __launch_bounds__(256) k_lower_count(const u64* cand_child, uint16_t* cand_prefix, i64* cand_counts,
                                                     const int32_t* d_num_cands) {
  const i64 c = (i64)blockIdx.x * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (c >= *d_num_cands) return;  // uniform per wave
  const u64 w = cand_child[c * 64 + lane];
  const int cnt = popc64(w);
  const int inc = wave_incl_scan(cnt);
  cand_prefix[c * 64 + lane] = (uint16_t)(inc - cnt);
  if (lane == kWave - 1) cand_counts[c] = (i64)inc | ((i64)(inc > 0 ? 1 : 0) << 32);
}

__global__ void __launch_bounds__(256) k_tile_flags(const int32_t* tile_lower_base, const i64* cand_scan,
                                                    int32_t* tile_nonempty, const int32_t* d_num_tiles) {
  const i64 t = (i64)blockIdx.x * 256 + threadIdx.x;
  if (t >= *d_num_tiles) return;
  tile_nonempty[t] = scan_leaf(cand_scan[tile_lower_base[t + 1]]) > scan_leaf(cand_scan[tile_lower_base[t]]) ? 1 : 0;
}

// Per-grid counts and begins of grid g (shared by both launch shapes).
__device__ __forceinline__ void grid_counts_one(i64 g, const int32_t* grid_tile_begin, const int32_t* tile_lower_base,
                                                const int32_t* upper_excl, const i64* cand_scan, int32_t* grid_info,
                                                int32_t* readback) {
  const int32_t tb = grid_tile_begin[g], te = grid_tile_begin[g + 1];
  const i64 vb = cand_scan[tile_lower_base[tb]], ve = cand_scan[tile_lower_base[te]];
  const int32_t nu = upper_excl[te] - upper_excl[tb];
  const int32_t n1 = scan_lower(ve) - scan_lower(vb);
  const int32_t nl = scan_leaf(ve) - scan_leaf(vb);
  int32_t* gi = grid_info + g * 6;
  gi[0] = nu;
  gi[1] = n1;
  gi[2] = nl;
  gi[3] = upper_excl[tb];
  gi[4] = scan_lower(vb);
  gi[5] = scan_leaf(vb);
  readback[4 + g * 3 + 0] = nu;
  readback[4 + g * 3 + 1] = n1;
  readback[4 + g * 3 + 2] = nl;
}

__device__ __forceinline__ void batch_totals(const int32_t* upper_excl, const i64* cand_scan, int32_t nt, int32_t nc,
                                             int32_t* readback) {
  const i64 last = cand_scan[nc];
  readback[1] = upper_excl[nt];
  readback[2] = scan_lower(last);
  readback[3] = scan_leaf(last);
}

__global__ void __launch_bounds__(256) k_grid_counts(const int32_t* grid_tile_begin, const int32_t* tile_lower_base,
                                                     const int32_t* upper_excl, const i64* cand_scan,
                                                     const int32_t* d_num_tiles, const int32_t* d_num_cands, int32_t B,
                                                     int32_t* grid_info, int32_t* readback) {
  const i64 g = (i64)blockIdx.x * 256 + threadIdx.x;
  if (g == 0) batch_totals(upper_excl, cand_scan, *d_num_tiles, *d_num_cands, readback);
  if (g >= B) return;
  grid_counts_one(g, grid_tile_begin, tile_lower_base, upper_excl, cand_scan, grid_info, readback);
}

// Small batches (at most 4096 tiles): non-empty tile flags, their exclusive
// scan (output upper indices) and the per-grid counts in one workgroup.
constexpr int kTailThreads = 1024;
constexpr int kTailItems = 4;
constexpr int kTailTiles = kTailThreads * kTailItems;

// Stages tile_lower_base[0, cap_t] (cap_t <= kTailTiles, the tile capacity known
// to the host) in LDS. The loads do not wait for the tile count, and all of
// them are in flight at once (clamped indices, no conditional load).
__device__ __forceinline__ void stage_tile_bases(const int32_t* tile_lower_base, int32_t cap_t, int32_t* s_tlb) {
  int32_t v[kTailItems + 1];
#pragma unroll
  for (int k = 0; k <= kTailItems; ++k) v[k] = tile_lower_base[min(k * kTailThreads + (int)threadIdx.x, cap_t)];
#pragma unroll
  for (int k = 0; k <= kTailItems; ++k) {
    const int t = k * kTailThreads + threadIdx.x;
    if (t <= cap_t) s_tlb[t] = v[k];
  }
}

// Tile t (< nt) is non-empty when its candidate lowers hold a leaf. s_tlb holds
// the tiles' candidate bases (staged, the caller has synchronised), cs the
// packed candidate scan (LDS or global), gt the grid_tile_begin pair of grid
// threadIdx.x (loaded early by the caller). Upper indices stay in LDS (s_uex) for
// the per-grid counts and go to upper_excl for the node writers.
__device__ __forceinline__ void counts_tail_body(const int32_t* grid_tile_begin, int2 gt, const int32_t* s_tlb,
                                                 const i64* cs, int32_t nt, int32_t nc, int32_t B, int32_t* s_uex,
                                                 int32_t* upper_excl, int32_t* grid_info, int32_t* readback,
                                                 int32_t* s_wave, int32_t* host_rb) {
  const int tid = threadIdx.x;
  int32_t lv[kTailItems + 1];
#pragma unroll
  for (int k = 0; k <= kTailItems; ++k) lv[k] = scan_leaf(cs[s_tlb[min(tid * kTailItems + k, nt)]]);
  int f[kTailItems];
  int sum = 0;
#pragma unroll
  for (int k = 0; k < kTailItems; ++k) {
    f[k] = tid * kTailItems + k < nt && lv[k + 1] > lv[k] ? 1 : 0;
    sum += f[k];
  }
  int total;
  int ex = block_excl_scan<int, kTailThreads>(sum, s_wave, total);
#pragma unroll
  for (int k = 0; k < kTailItems; ++k) {
    const int t = tid * kTailItems + k;
    if (t < nt) {
      s_uex[t] = ex;
      upper_excl[t] = ex;
    }
    ex += f[k];
  }
  if (tid == 0) {
    s_uex[nt] = total;
    upper_excl[nt] = total;
    const i64 last = cs[nc];
    readback[1] = total;
    readback[2] = scan_lower(last);
    readback[3] = scan_leaf(last);
    if (host_rb) {  // the flag word as the earlier launches left it (this one sets none)
      host_rb[0] = readback[0];
      host_rb[1] = total;
      host_rb[2] = scan_lower(last);
      host_rb[3] = scan_leaf(last);
    }
  }
  __syncthreads();
  for (int32_t g = tid; g < B; g += kTailThreads) {
    const int32_t tb = g == tid ? gt.x : grid_tile_begin[g], te = g == tid ? gt.y : grid_tile_begin[g + 1];
    const i64 vb = cs[s_tlb[tb]], ve = cs[s_tlb[te]];
    const int32_t nu = s_uex[te] - s_uex[tb];
    const int32_t n1 = scan_lower(ve) - scan_lower(vb);
    const int32_t nl = scan_leaf(ve) - scan_leaf(vb);
    int32_t* gi = grid_info + (i64)g * 6;
    gi[0] = nu;
    gi[1] = n1;
    gi[2] = nl;
    gi[3] = s_uex[tb];
    gi[4] = scan_lower(vb);
    gi[5] = scan_leaf(vb);
    readback[4 + g * 3 + 0] = nu;
    readback[4 + g * 3 + 1] = n1;
    readback[4 + g * 3 + 2] = nl;
    if (host_rb) {
      host_rb[4 + g * 3 + 0] = nu;
      host_rb[4 + g * 3 + 1] = n1;
      host_rb[4 + g * 3 + 2] = nl;
    }
  }
}

__device__ __forceinline__ int2 load_grid_tiles(const int32_t* grid_tile_begin, int32_t B) {
  const int g = min((int)threadIdx.x, B);  // grid_tile_begin has B + 1 entries
  return make_int2(grid_tile_begin[g], grid_tile_begin[min(g + 1, B)]);
}

__global__ void __launch_bounds__(kTailThreads) k_counts_tail(const int32_t* grid_tile_begin,
                                                              const int32_t* tile_lower_base, int32_t cap_t,
                                                              const i64* cand_scan, const int32_t* d_num_tiles,
                                                              const int32_t* d_num_cands, int32_t B,
                                                              int32_t* upper_excl, int32_t* grid_info,
                                                              int32_t* readback, int32_t* host_rb) {
  __shared__ int32_t s_tlb[kTailTiles + 1];
  __shared__ int32_t s_uex[kTailTiles + 1];
  __shared__ int32_t s_wave[kTailThreads / kWave];
  const int32_t nt = *d_num_tiles, nc = *d_num_cands;
  const int2 gt = load_grid_tiles(grid_tile_begin, B);
  stage_tile_bases(tile_lower_base, cap_t, s_tlb);
  __syncthreads();
  counts_tail_body(grid_tile_begin, gt, s_tlb, cand_scan, nt, nc, B, s_uex, upper_excl, grid_info, readback, s_wave,
                   host_rb);
}

// Up to kScanTailMax candidates whose packed counts the marking wrote: the
// scan of the counts and the tail above in one workgroup (one launch instead of
// two; the tail reads the scan this workgroup wrote, after a block barrier).
constexpr i64 kScanTailMax = 65536;

__global__ void __launch_bounds__(kTailThreads) k_scan_counts_tail(const i64* cand_counts, i64* cand_scan,
                                                                   int32_t cap_c, const int32_t* grid_tile_begin,
                                                                   const int32_t* tile_lower_base, int32_t cap_t,
                                                                   const int32_t* d_num_tiles,
                                                                   const int32_t* d_num_cands, int32_t B,
                                                                   int32_t* upper_excl, int32_t* grid_info,
                                                                   int32_t* readback, int32_t* host_rb) {
  __shared__ int32_t s_tlb[kTailTiles + 1];
  __shared__ int32_t s_uex[kTailTiles + 1];
  __shared__ int32_t s_wave[kTailThreads / kWave];
  __shared__ i64 s_wave64[kTailThreads / kWave];
  const int32_t nt = *d_num_tiles;
  const int32_t nc = min(max(*d_num_cands, 0), cap_c);
  const int2 gt = load_grid_tiles(grid_tile_begin, B);
  stage_tile_bases(tile_lower_base, cap_t, s_tlb);
  block_scan_all<i64, kTailThreads, 8>(cand_counts, cand_scan, nc, nullptr, s_wave64);
  __syncthreads();  // the scan is read below, by this workgroup only
  counts_tail_body(grid_tile_begin, gt, s_tlb, cand_scan, nt, nc, B, s_uex, upper_excl, grid_info, readback, s_wave,
                   host_rb);
}

// Small batches (at most kCountsSmallMax candidates and kTailTiles tiles):
// candidate leaf counts and prefix tables, their packed scan and the tail above,
// in one workgroup. Every global load (the counts, the candidate masks up to
// the host-known capacity cap_c, the tile bases, the grid ranges) is issued
// before the first wait.
constexpr int kCountsSmallMax = 4096;

__global__ void __launch_bounds__(kTailThreads) k_counts_small(const u64* cand_child, int32_t cap_c,
                                                               uint16_t* cand_prefix, i64* cand_counts,
                                                               i64* cand_scan, const int32_t* grid_tile_begin,
                                                               const int32_t* tile_lower_base, int32_t cap_t,
                                                               const int32_t* d_num_tiles,
                                                               const int32_t* d_num_cands, int32_t B,
                                                               int32_t* upper_excl, int32_t* grid_info,
                                                               int32_t* readback, int counts_ready,
                                                               int32_t* host_rb) {
  __shared__ i64 s_cc[kCountsSmallMax + 1];
  __shared__ int32_t s_tlb[kTailTiles + 1];
  __shared__ int32_t s_uex[kTailTiles + 1];
  __shared__ int32_t s_wave[kTailThreads / kWave];
  __shared__ i64 s_wave64[kTailThreads / kWave];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int32_t nc = *d_num_cands;
  const int32_t nt = *d_num_tiles;
  const int2 gt = load_grid_tiles(grid_tile_begin, B);
  stage_tile_bases(tile_lower_base, cap_t, s_tlb);
  // one wave per candidate, up to 2048 / 16 = 128 per wave: per-word prefix and
  // the packed count. The masks are loaded up to the capacity (clamped), so no
  // load waits for the candidate count.
  constexpr int kWaves = kTailThreads / kWave;
  constexpr int kPerWave = 4;
  if (counts_ready) {  // prefixes and counts came with the masks
    for (int c = tid; c < nc; c += kTailThreads) s_cc[c] = cand_counts[c];
  }
  for (int c0 = wv * kPerWave; !counts_ready && c0 < cap_c; c0 += kWaves * kPerWave) {
    u64 w[kPerWave];
#pragma unroll
    for (int v = 0; v < kPerWave; ++v) w[v] = cand_child[(i64)min(c0 + v, cap_c - 1) * 64 + lane];
#pragma unroll
    for (int v = 0; v < kPerWave; ++v) {
      if (c0 + v >= nc) break;
      const int cnt = popc64(w[v]);
      const int inc = wave_incl_scan(cnt);
      cand_prefix[(i64)(c0 + v) * 64 + lane] = (uint16_t)(inc - cnt);
      if (lane == kWave - 1) {
        const i64 packed = (i64)inc | ((i64)(inc > 0 ? 1 : 0) << 32);
        cand_counts[c0 + v] = packed;
        s_cc[c0 + v] = packed;
      }
    }
  }
  __syncthreads();
  // exclusive scan of the packed counts (blocked, 2 per thread)
  constexpr int kPer = kCountsSmallMax / kTailThreads;
  i64 v[kPer];
  i64 sum = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int c = tid * kPer + k;
    v[k] = c < nc ? s_cc[c] : 0;
    sum += v[k];
  }
  i64 total;
  i64 ex = block_excl_scan<i64, kTailThreads>(sum, s_wave64, total);
  // every thread has read its counts from s_cc (the scan's barriers), so the
  // scan can replace them in LDS for the tail below
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int c = tid * kPer + k;
    if (c < nc) {
      cand_scan[c] = ex;
      s_cc[c] = ex;
    }
    ex += v[k];
  }
  if (tid == 0) {
    cand_scan[nc] = total;
    s_cc[nc] = total;
  }
  __syncthreads();
  counts_tail_body(grid_tile_begin, gt, s_tlb, s_cc, nt, nc, B, s_uex, upper_excl, grid_info, readback, s_wave,
                   host_rb);
}

bool tree_counts(TreeScratch& ts, int32_t B, hipStream_t s, int32_t* host_rb) {
  if (ts.cap_cands <= kCountsSmallMax && ts.cap_tiles <= (i64)kTailThreads * kTailItems) {
    launch("k_counts_small", k_counts_small, 1, kTailThreads, s, (const u64*)ts.cand_child, (int32_t)ts.cap_cands,
           ts.cand_prefix, ts.cand_counts, ts.cand_scan, (const int32_t*)ts.grid_tile_begin,
           (const int32_t*)ts.tile_lower_base, (int32_t)ts.cap_tiles, (const int32_t*)ts.d_num_tiles,
           (const int32_t*)ts.d_num_cands, B, ts.upper_excl, ts.grid_info, ts.readback,
           ts.cand_counts_ready ? 1 : 0, host_rb);
    return host_rb != nullptr;
  }
  if (ts.cand_counts_ready && ts.cap_cands <= kScanTailMax && ts.cap_tiles <= (i64)kTailTiles) {
    launch("k_scan_counts_tail", k_scan_counts_tail, 1, kTailThreads, s, (const i64*)ts.cand_counts,
           ts.cand_scan, (int32_t)ts.cap_cands, (const int32_t*)ts.grid_tile_begin,
           (const int32_t*)ts.tile_lower_base, (int32_t)ts.cap_tiles, (const int32_t*)ts.d_num_tiles,
           (const int32_t*)ts.d_num_cands, B, ts.upper_excl, ts.grid_info, ts.readback, host_rb);
    return host_rb != nullptr;
  }
  tree_count_cands(ts, s);
  return tree_grid_counts(ts, B, s, host_rb);
}

void tree_count_cands(TreeScratch& ts, hipStream_t s) {
  if (!ts.cand_counts_ready)
    launch("k_lower_count", k_lower_count, ceil_div(ts.cap_cands, 4), 256, s, (const u64*)ts.cand_child,
           ts.cand_prefix, ts.cand_counts, (const int32_t*)ts.d_num_cands);
  scan_excl_i64(ts.cand_counts, ts.cand_scan, ts.cap_cands, ts.d_num_cands, s, nullptr, ts.scan_tmp);
}

bool tree_grid_counts(TreeScratch& ts, int32_t B, hipStream_t s, int32_t* host_rb) {
  if (ts.cap_tiles <= (i64)kTailThreads * kTailItems) {
    launch("k_counts_tail", k_counts_tail, 1, kTailThreads, s, (const int32_t*)ts.grid_tile_begin,
           (const int32_t*)ts.tile_lower_base, (int32_t)ts.cap_tiles, (const i64*)ts.cand_scan,
           (const int32_t*)ts.d_num_tiles, (const int32_t*)ts.d_num_cands, B, ts.upper_excl, ts.grid_info,
           ts.readback, host_rb);
    return host_rb != nullptr;
  }
  launch("k_tile_flags", k_tile_flags, ceil_div(ts.cap_tiles, 256), 256, s, (const int32_t*)ts.tile_lower_base,
         (const i64*)ts.cand_scan, ts.tile_nonempty, (const int32_t*)ts.d_num_tiles);
  scan_excl_i32(ts.tile_nonempty, ts.upper_excl, ts.cap_tiles, ts.d_num_tiles, s, nullptr, ts.scan_tmp);
  launch("k_grid_counts", k_grid_counts, ceil_div((i64)B, 256), 256, s, (const int32_t*)ts.grid_tile_begin,
         (const int32_t*)ts.tile_lower_base, (const int32_t*)ts.upper_excl, (const i64*)ts.cand_scan,
         (const int32_t*)ts.d_num_tiles, (const int32_t*)ts.d_num_cands, B, ts.grid_info, ts.readback);
  return false;
}

// ------------------------------------------------------------------ node writers
constexpr int kNodeFlags = 4096;  // candidates per tile whose non-empty flags the tile block stages in LDS
constexpr int kNodesDense = 1024;  // leaves of a candidate from which the node writer goes word by word
// One launch, two roles. Blocks [0, tile_blocks) each own one tile and write its
// upper node record and child mask (candidate bits whose lower turned out empty
// are cleared). The remaining blocks own four candidate lowers each (one wave
// per candidate) and write the lower node record plus one leaf record (origin,
// grid, parent) per set bit of its leaf mask; leaf_cand[leaf] remembers the
// candidate for the leaf-mask producers. Block 0 also sets every header's box
// to empty for the leaf finalizer.
// cand_scan and upper_excl may point into LDS (the fused writer below, kLdsScan):
// then a candidate's leaf count and non-empty flag come from its two scan
// entries, and no count is loaded.
template <bool kLdsScan>
__device__ __forceinline__ void write_nodes_body(
    int32_t tile_blocks, const int4* utile, const u64* tile_child, const uint16_t* tile_prefix,
    const int32_t* tile_lower_base, const int4* cand_origin, const u64* cand_child, const uint16_t* cand_prefix,
    const i64* cand_counts, const i64* cand_scan, const int32_t* upper_excl, const int32_t* d_num_tiles,
    const int32_t* d_num_cands, int32_t n_upper, int32_t n_lower, int32_t n_leaf, int4* upper_origin,
    u64* upper_key, int32_t* upper_first, u64* upper_mask, int4* lower_origin, int32_t* lower_first,
    u64* lower_mask, uint16_t* lower_prefix, int4* leaf_origin, int32_t* leaf_parent, int32_t* leaf_cand,
    tc_grid_header* hdr, int32_t B, i64 cap_cands, uint32_t* s_flags) {
  if (blockIdx.x == 0) {  // every grid's box starts empty; the leaf finalizer folds into it
    for (int32_t g = threadIdx.x; g < B; g += 256) {
      for (int a = 0; a < 3; ++a) {
        hdr[g].bbox_min[a] = INT32_MAX;
        hdr[g].bbox_max[a] = INT32_MIN;
      }
    }
  }
  if ((int32_t)blockIdx.x < tile_blocks) {
    // every load indexed by the tile alone first (t < the tile capacity), then
    // the two scan entries they select
    const i64 t = blockIdx.x;
    const int32_t nt = *d_num_tiles;
    const int32_t cb = tile_lower_base[t], ce = tile_lower_base[t + 1];
    const i64 u = upper_excl[t];
    const int4 T = utile[t];
    u64 words[2];
    uint16_t pres[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      words[k] = tile_child[t * 512 + threadIdx.x * 2 + k];
      pres[k] = tile_prefix[t * 512 + threadIdx.x * 2 + k];
    }
    if (t >= nt) return;
    const i64 vb = cand_scan[cb];
    if (scan_leaf(cand_scan[ce]) == scan_leaf(vb)) return;  // empty tile, uniform per block
    if (u < 0 || u >= n_upper) return;  // cannot happen for consistent counts
    if (threadIdx.x == 0) {
      upper_origin[u] = make_int4(T.x * 4096, T.y * 4096, T.z * 4096, T.w);
      upper_key[u] = ((u64)(T.x + kTileBias) << 40) | ((u64)(T.y + kTileBias) << 20) | (u64)(T.z + kTileBias);
      upper_first[u] = scan_lower(vb);
    }
    // the tile's candidates' non-empty flags as an LDS bitset (loads of up to
    // kNodeFlags candidates in flight together), so that the per-bit loop below
    // waits on no memory; tiles with more candidates read the counts directly
    const int32_t ncb = ce - cb;
    const bool lds_flags = !kLdsScan && ncb <= kNodeFlags;  // uniform
    if (lds_flags) {
      const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
      for (int q = 0; q < kNodeFlags / 256; ++q) {
        const int32_t k = q * 256 + threadIdx.x;
        const bool ne = k < ncb && (int32_t)cand_counts[cb + min(k, ncb - 1)] > 0;
        const u64 bal = __ballot(ne);
        if (lane == 0) {
          s_flags[k >> 5] = (uint32_t)bal;
          s_flags[(k >> 5) + 1] = (uint32_t)(bal >> 32);
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int w = threadIdx.x * 2 + k;
      u64 word = words[k];
      u64 out = 0;
      int32_t c = pres[k];  // candidate index relative to the tile's base
      while (word) {
        const int b = __builtin_ctzll(word);
        bool ne;
        if constexpr (kLdsScan) ne = scan_leaf(cand_scan[cb + c + 1]) > scan_leaf(cand_scan[cb + c]);
        else ne = lds_flags ? ((s_flags[c >> 5] >> (c & 31)) & 1u) != 0 : (int32_t)cand_counts[cb + c] > 0;
        if (ne) out |= 1ull << b;
        word &= word - 1;
        ++c;
      }
      upper_mask[u * 512 + w] = out;
    }
    return;
  }
  // Candidate waves loop over the candidates (wave k takes k, k + K, ... for K
  // candidate waves in the launch, which may be fewer than the capacity), so no
  // wave runs for a candidate past the device count. Per candidate, every load
  // indexed by the candidate alone first (clamped to the capacity), then the two
  // that its origin selects.
  const int lane = threadIdx.x & (kWave - 1);
  const int32_t ncand = *d_num_cands;
  const i64 nstride = ((i64)gridDim.x - tile_blocks) * 4;
  for (i64 c = ((i64)blockIdx.x - tile_blocks) * 4 + threadIdx.x / kWave; c < ncand; c += nstride) {
    const i64 cc = c < cap_cands ? c : cap_cands - 1;
    const i64 v = cand_scan[cc];
    const int32_t cnt = kLdsScan ? scan_leaf(cand_scan[cc + 1]) - scan_leaf(v) : (int32_t)cand_counts[cc];
    const int4 co = cand_origin[cc];
    const u64 word = cand_child[cc * 64 + lane];
    const uint16_t pre = cand_prefix[cc * 64 + lane];
    if (c >= cap_cands) break;  // cannot happen for a consistent count
    if (cnt == 0) continue;  // uniform per wave
    const i64 lo = scan_lower(v);
    const int32_t lb = scan_leaf(v);
    if (lo < 0 || lo >= n_lower || lb < 0 || (i64)lb + cnt > n_leaf) continue;  // consistency guard
    const int32_t g = utile[co.w].w;
    lower_mask[lo * 64 + lane] = word;
    lower_prefix[lo * 64 + lane] = pre;
    if (lane == 0) {
      lower_origin[lo] = make_int4(co.x, co.y, co.z, upper_excl[co.w]);
      lower_first[lo] = lb;
    }
    // leaf records in output order, 64 at a time: lane j takes leaf r = k0 + j, finds
    // its word (last word whose prefix is <= r, by binary search over the lanes'
    // prefixes) and bit, so consecutive lanes store consecutive records
    // Dense candidates (at least kNodesDense leaves) go word by word instead:
    // for each non-empty word j (a wave-uniform loop), lane l writes the record
    // of its l-th set bit, so no lane searches (a full word needs no select).
    const int pre_i = pre;
    auto put = [&](int r, int bit) {
      const int px = bit >> 8, py = (bit >> 4) & 15, pz = bit & 15;
      const i64 idx = (i64)lb + r;
      leaf_origin[idx] = make_int4(co.x + px * 8, co.y + py * 8, co.z + pz * 8, g);
      leaf_parent[idx] = (int32_t)lo;
      leaf_cand[idx] = (int32_t)c;
    };
    if (cnt >= kNodesDense) {  // uniform
      u64 ne = (u64)__ballot(word != 0);
      while (ne) {
        const int j = __builtin_ctzll(ne);
        ne &= ne - 1;
        const u64 wj = ((u64)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(word >> 32), j) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)word, j);
        const int pj = __builtin_amdgcn_readlane(pre_i, j);
        const int pc = popc64(wj);
        if (lane < pc) put(pj + lane, j * 64 + (pc == 64 ? lane : select_bit(wj, lane)));
      }
      continue;
    }
    for (int32_t k0 = 0; k0 < cnt; k0 += kWave) {
      const int32_t r = k0 + lane;
      int w = 0;
#pragma unroll
      for (int step = 32; step >= 1; step >>= 1) {
        const int p = __shfl(pre_i, w + step, kWave);
        if (w + step < kWave && p <= r) w += step;
      }
      const u64 ww = __shfl(word, w, kWave);
      const int pw = __shfl(pre_i, w, kWave);
      if (r >= cnt) continue;
      put(r, w * 64 + select_bit(ww, r - pw));  // bit (x*16 + y)*16 + z
    }
  }
}

__global__ void __launch_bounds__(256) k_write_nodes(
    int32_t tile_blocks, const int4* utile, const u64* tile_child, const uint16_t* tile_prefix,
    const int32_t* tile_lower_base, const int4* cand_origin, const u64* cand_child, const uint16_t* cand_prefix,
    const i64* cand_counts, const i64* cand_scan, const int32_t* upper_excl, const int32_t* d_num_tiles,
    const int32_t* d_num_cands, int32_t n_upper, int32_t n_lower, int32_t n_leaf, int4* upper_origin,
    u64* upper_key, int32_t* upper_first, u64* upper_mask, int4* lower_origin, int32_t* lower_first,
    u64* lower_mask, uint16_t* lower_prefix, int4* leaf_origin, int32_t* leaf_parent, int32_t* leaf_cand,
    tc_grid_header* hdr, int32_t B, i64 cap_cands) {
  __shared__ uint32_t s_flags[kNodeFlags / 32];
  write_nodes_body<false>(tile_blocks, utile, tile_child, tile_prefix, tile_lower_base, cand_origin, cand_child, cand_prefix,
                   cand_counts, cand_scan, upper_excl, d_num_tiles, d_num_cands, n_upper, n_lower, n_leaf,
                   upper_origin, upper_key, upper_first, upper_mask, lower_origin, lower_first, lower_mask,
                   lower_prefix, leaf_origin, leaf_parent, leaf_cand, hdr, B, cap_cands, s_flags);
}

// Small batches whose marking wrote the candidates' packed counts (at most
// kWnCands candidates and kWnTiles tiles): the counts stage and the node writer
// in one launch, which saves the host one launch per pass. Every working block
// first scans the packed counts and the tiles' non-empty flags itself, into LDS
// (a few KB of loads, all in flight together), so no block waits on another;
// block 0 also writes the per-grid counts and begins (grid_info) and the batch
// totals (readback) that the later stages read. Blocks past the live tiles and
// candidates leave first.
constexpr int kWnCands = 2048;
constexpr int kWnTiles = 2048;
constexpr int kWnPer = kWnCands / 256;
static_assert(kWnTiles / 256 == kWnPer, "one item count for both scans");

__global__ void __launch_bounds__(256) k_write_nodes_counted(
    int32_t tile_blocks, const int4* utile, const u64* tile_child, const uint16_t* tile_prefix,
    const int32_t* tile_lower_base, const int4* cand_origin, const u64* cand_child, const uint16_t* cand_prefix,
    const i64* cand_counts, const int32_t* d_num_tiles, const int32_t* d_num_cands, int32_t n_upper,
    int32_t n_lower, int32_t n_leaf, int4* upper_origin, u64* upper_key, int32_t* upper_first, u64* upper_mask,
    int4* lower_origin, int32_t* lower_first, u64* lower_mask, uint16_t* lower_prefix, int4* leaf_origin,
    int32_t* leaf_parent, int32_t* leaf_cand, tc_grid_header* hdr, int32_t B, i64 cap_cands,
    const int32_t* grid_tile_begin, int32_t* grid_info, int32_t* readback) {
  __shared__ i64 s_cc[kWnCands + 1];
  __shared__ int32_t s_tlb[kWnTiles + 1];
  __shared__ int32_t s_uex[kWnTiles + 1];
  __shared__ i64 s_wave64[256 / kWave];
  __shared__ int32_t s_wave[256 / kWave];
  __shared__ uint32_t s_flags[kNodeFlags / 32];
  const int tid = threadIdx.x;
  const int32_t cap_c = (int32_t)cap_cands, cap_t = tile_blocks;
  // every load first, at clamped indices (the counts up to the capacities)
  i64 v[kWnPer];
  int32_t tb[kWnPer + 1];
#pragma unroll
  for (int k = 0; k < kWnPer; ++k) v[k] = cand_counts[min(tid * kWnPer + k, cap_c - 1)];
#pragma unroll
  for (int k = 0; k <= kWnPer; ++k) tb[k] = tile_lower_base[min(tid * kWnPer + k, cap_t)];
  int32_t nt = *d_num_tiles, nc = *d_num_cands;
  if (nt < 0 || nt > cap_t || nc < 0 || nc > cap_c) {  // consistency guard (the LDS holds the capacities)
    if (blockIdx.x == 0 && tid == 0) atomicOr(&readback[0], kFlagInternal);
    nt = min(max(nt, 0), cap_t);
    nc = min(max(nc, 0), cap_c);
  }
  const int32_t bx = blockIdx.x;
  if (bx != 0 && (bx < tile_blocks ? bx >= nt : (i64)(bx - tile_blocks) * 4 >= nc)) return;  // uniform
  // exclusive scan of the packed counts: a candidate's first leaf and output lower
  i64 sum = 0;
#pragma unroll
  for (int k = 0; k < kWnPer; ++k) {
    if (tid * kWnPer + k >= nc) v[k] = 0;
    sum += v[k];
  }
  i64 total;
  i64 ex = block_excl_scan<i64, 256>(sum, s_wave64, total);
#pragma unroll
  for (int k = 0; k < kWnPer; ++k) {
    const int c = tid * kWnPer + k;
    if (c < nc) s_cc[c] = ex;
    ex += v[k];
  }
  if (tid == 0) s_cc[nc] = total;
#pragma unroll
  for (int k = 0; k <= kWnPer; ++k) {
    const int t = tid * kWnPer + k;
    if (t <= nt) s_tlb[t] = tb[k];
  }
  __syncthreads();
  // non-empty tiles and their exclusive scan: the output upper indices
  int f[kWnPer];
  int fsum = 0;
#pragma unroll
  for (int k = 0; k < kWnPer; ++k) {
    const int t = tid * kWnPer + k;
    f[k] = t < nt && scan_leaf(s_cc[s_tlb[t + 1]]) > scan_leaf(s_cc[s_tlb[t]]) ? 1 : 0;
    fsum += f[k];
  }
  int nu;
  int fex = block_excl_scan<int, 256>(fsum, s_wave, nu);
#pragma unroll
  for (int k = 0; k < kWnPer; ++k) {
    const int t = tid * kWnPer + k;
    if (t < nt) s_uex[t] = fex;
    fex += f[k];
  }
  if (tid == 0) s_uex[nt] = nu;
  __syncthreads();
  if (bx == 0) {  // per-grid counts and begins, batch totals
    if (tid == 0) {
      readback[1] = nu;
      readback[2] = scan_lower(s_cc[nc]);
      readback[3] = scan_leaf(s_cc[nc]);
    }
    for (int32_t g = tid; g < B; g += 256) {
      const int32_t t0 = grid_tile_begin[g], t1 = grid_tile_begin[g + 1];
      const i64 vb = s_cc[s_tlb[t0]], ve = s_cc[s_tlb[t1]];
      const int32_t nug = s_uex[t1] - s_uex[t0];
      const int32_t n1 = scan_lower(ve) - scan_lower(vb);
      const int32_t nl = scan_leaf(ve) - scan_leaf(vb);
      int32_t* gi = grid_info + (i64)g * 6;
      gi[0] = nug;
      gi[1] = n1;
      gi[2] = nl;
      gi[3] = s_uex[t0];
      gi[4] = scan_lower(vb);
      gi[5] = scan_leaf(vb);
      readback[4 + g * 3 + 0] = nug;
      readback[4 + g * 3 + 1] = n1;
      readback[4 + g * 3 + 2] = nl;
    }
  }
  write_nodes_body<true>(tile_blocks, utile, tile_child, tile_prefix, tile_lower_base, cand_origin, cand_child,
                         cand_prefix, cand_counts, s_cc, s_uex, d_num_tiles, d_num_cands, n_upper, n_lower, n_leaf, upper_origin,
                   upper_key, upper_first, upper_mask, lower_origin, lower_first, lower_mask, lower_prefix,
                   leaf_origin, leaf_parent, leaf_cand, hdr, B, cap_cands, s_flags);
}

bool write_nodes_counted_fits(const TreeScratch& ts, int32_t B) {
  return ts.cand_counts_ready && ts.cap_cands >= 1 && ts.cap_cands <= kWnCands && ts.cap_tiles >= 1 &&
         ts.cap_tiles <= kWnTiles && B >= 1;
}

void tree_write_nodes_counted(TreeScratch& ts, const GridView& out, int32_t* leaf_cand, hipStream_t s) {
  if (!write_nodes_counted_fits(ts, out.B)) throw Error(TC_ERR_INTERNAL, "nodes: too many candidates for one launch");
  const i64 tile_blocks = ts.cap_tiles;
  launch("k_write_nodes", k_write_nodes_counted, tile_blocks + ceil_div(ts.cap_cands, 4), 256, s,
         (int32_t)tile_blocks, (const int4*)ts.utile, (const u64*)ts.tile_child, (const uint16_t*)ts.tile_prefix,
         (const int32_t*)ts.tile_lower_base, (const int4*)ts.cand_origin, (const u64*)ts.cand_child,
         (const uint16_t*)ts.cand_prefix, (const i64*)ts.cand_counts, (const int32_t*)ts.d_num_tiles,
         (const int32_t*)ts.d_num_cands, out.n_upper, out.n_lower, out.n_leaf, out.upper_origin, out.upper_key,
         out.upper_first, out.upper_mask, out.lower_origin, out.lower_first, out.lower_mask, out.lower_prefix,
         out.leaf_origin, out.leaf_parent, leaf_cand, out.headers, out.B, ts.cap_cands,
         (const int32_t*)ts.grid_tile_begin, ts.grid_info, ts.readback);
}

void tree_write_nodes(TreeScratch& ts, const GridView& out, int32_t* leaf_cand, hipStream_t s) {
  const i64 tile_blocks = ts.cap_tiles;
  // candidate workgroups: one resident round at most (the waves loop over the candidates)
  const i64 cand_blocks = std::min(ceil_div(ts.cap_cands, 4), (i64)device_cu_count() * 8);
  launch("k_write_nodes", k_write_nodes, tile_blocks + cand_blocks, 256, s, (int32_t)tile_blocks,
         (const int4*)ts.utile, (const u64*)ts.tile_child, (const uint16_t*)ts.tile_prefix,
         (const int32_t*)ts.tile_lower_base, (const int4*)ts.cand_origin, (const u64*)ts.cand_child,
         (const uint16_t*)ts.cand_prefix, (const i64*)ts.cand_counts, (const i64*)ts.cand_scan,
         (const int32_t*)ts.upper_excl, (const int32_t*)ts.d_num_tiles, (const int32_t*)ts.d_num_cands, out.n_upper,
         out.n_lower, out.n_leaf, out.upper_origin, out.upper_key, out.upper_first, out.upper_mask, out.lower_origin,
         out.lower_first, out.lower_mask, out.lower_prefix, out.leaf_origin, out.leaf_parent, leaf_cand, out.headers,
         out.B, ts.cap_cands);
}

// ------------------------------------------------------------------ leaf statistics
// Per leaf (masks built by the ijk front-end as eight word slices, slice k
// holding word k of every leaf): the leaf mask, prefix word, voxel count and
// packed local bbox. The topology pass computes the same values in its gather.
__global__ void __launch_bounds__(256) k_leaf_stats(const u64* slices, u64* leaf_mask, u64* leaf_prefix,
                                                    uint32_t* leaf_box, int32_t* leaf_inrun, i64* vox_part,
                                                    i64 n_leaf) {
  const i64 i = (i64)blockIdx.x * 256 + threadIdx.x;
  int count = 0;
  u64 prefix = 0;
  uint32_t box = kEmptyBox;
  if (i < n_leaf) {
    u64 W[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) W[k] = slices[k * n_leaf + i];
#pragma unroll
    for (int k = 0; k < 8; k += 2) reinterpret_cast<ulonglong2*>(leaf_mask)[i * 4 + k / 2] = make_ulonglong2(W[k], W[k + 1]);
    leaf_stats(W, prefix, count, box);
  }
  const int32_t inrun = block_run_scan(count, &vox_part[blockIdx.x]);
  if (i < n_leaf) {
    leaf_prefix[i] = prefix;
    leaf_box[i] = box;
    leaf_inrun[i] = inrun;
  }
}

void tree_leaf_stats(const GridView& out, const u64* slices, uint32_t* leaf_box, int32_t* leaf_inrun, i64* vox_part,
                     hipStream_t s) {
  launch("k_leaf_stats", k_leaf_stats, ceil_div((i64)out.n_leaf, 256), 256, s, slices, out.leaf_mask,
         out.leaf_prefix, leaf_box, leaf_inrun, vox_part, (i64)out.n_leaf);
}

// Per-grid bboxes of large batches: leaf bounds are reduced over the wave (leaves
// are sorted by grid, so a wave nearly always holds one grid) and then folded
// with device-scope atomics into one of R replicas of the per-grid accumulators,
// chosen by block. On this multi-XCD part such atomics resolve past the per-XCD
// L2 and serialize per address, so spreading them over replicas keeps each
// address cold; the header writer folds the replicas.
__device__ __forceinline__ void box_flush(int32_t* bbox, int32_t B, int32_t R, int rep, int g, const int v[6]) {
  if (g < 0 || g >= B) return;
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    atomicMin(&bbox[((i64)a * R + rep) * B + g], v[a]);
    atomicMax(&bbox[((i64)(3 + a) * R + rep) * B + g], v[3 + a]);
  }
}

int32_t bbox_replicas(int32_t B) {
  int32_t r = 8192 / (B > 0 ? B : 1);
  return r < 1 ? 1 : (r > 64 ? 64 : r);
}

// Small batches (at most kFinSmallLeaves leaves, kFinSmallGrids grids and
// kFinRuns runs): leaf offsets, bboxes and headers in one launch of
// ceil(L / kFinSlice) workgroups. The leaf producer left, per run of `gran`
// leaves, the run's voxel sum and every leaf's voxels before it inside its run.
// Every workgroup scans the (at most kFinRuns) run sums itself, so each run's
// offset is known without a second launch; a grid's voxel begin is its first
// leaf's run offset plus that leaf's in-run count. Each workgroup then writes
// the offsets of its kFinSlice leaves (wave w: a contiguous run of kFinPer * 64),
// folds their boxes per grid in LDS, and then into the headers with one set of
// atomics per grid it touched (the node writer has set every box to empty);
// workgroup 0 writes the other header fields. Totals stay below 2^31 here (L * 512 <= 2^27), so offsets
// are computed in 32 bits. All global loads that do not depend on another are
// issued first, at clamped indices.
constexpr int kFinThreads = 256;
constexpr int kFinPer = 8;
constexpr int kFinSlice = kFinThreads * kFinPer;  // leaves per workgroup
constexpr int kFinRuns = 4096;
constexpr i64 kFinSmallLeaves = 262144;  // totals below 2^31 voxels (512 per leaf)
constexpr int kFinSmallGrids = 1024;

__device__ __forceinline__ void box_fold_lds(int32_t (*s_box)[kFinSmallGrids], int g, const int v[6]) {
  for (int a = 0; a < 3; ++a) {
    atomicMin(&s_box[a][g], v[a]);
    atomicMax(&s_box[3 + a][g], v[3 + a]);
  }
}

__device__ __forceinline__ void finalize_small_body(const int4* leaf_origin, const int32_t* leaf_inrun,
                                                    const uint32_t* leaf_box, const i64* vox_part, int32_t gs,
                                                    const int32_t* grid_info, i64* leaf_offset, int32_t B,
                                                    const int32_t* d_L, int32_t L_cap, tc_grid_header* hdr,
                                                    int32_t* flags, int32_t* status, int32_t* host_words) {
  constexpr int kR = kFinRuns / kFinThreads;
  constexpr int kG = kFinSmallGrids / kFinThreads;
  // the leaf count from the device (the launch may be sized by a capacity):
  // workgroups past the leaves leave once it is in, block 0 always writes the
  // headers. The loads below are clamped to the capacity, so none waits for it.
  int32_t L = *d_L;
  const int32_t np_cap = (L_cap + (1 << gs) - 1) >> gs;  // runs of 2^gs leaves, by the capacity (>= 1)
  __shared__ int32_t s_part[kFinRuns];           // exclusive voxel offset of every run
  __shared__ int32_t s_gvb[kFinSmallGrids + 1];  // voxel begin of every grid, then the total
  __shared__ int32_t s_wave[kFinThreads / kWave];
  __shared__ int32_t s_box[6][kFinSmallGrids];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int32_t base = (int32_t)blockIdx.x * kFinSlice + (tid / kWave) * (kFinPer * kWave);  // this wave's run
  // block 0 writes the headers at the end: their node fields are loaded now, in
  // the first round of loads, rather than after the last barrier
  int32_t hv[kG][6];
  if (blockIdx.x == 0) {  // uniform
#pragma unroll
    for (int k = 0; k < kG; ++k) {
      const i64 gg = min(tid + k * kFinThreads, B - 1);  // B >= 1
#pragma unroll
      for (int f = 0; f < 6; ++f) hv[k][f] = grid_info[gg * 6 + f];
    }
  }
  const bool live = L_cap > 0;  // uniform; the launch holds ceil(L_cap / kFinSlice) workgroups, or one
  i64 pv[kR];
  int32_t gf[kG];
  int4 o[kFinPer];
  uint32_t bx[kFinPer];
  int32_t inr[kFinPer];
  if (live) {
#pragma unroll
    for (int k = 0; k < kR; ++k) pv[k] = vox_part[min(tid * kR + k, np_cap - 1)];
#pragma unroll
    for (int k = 0; k < kG; ++k) gf[k] = grid_info[(i64)min(tid * kG + k, B - 1) * 6 + 5];
#pragma unroll
    for (int k = 0; k < kFinPer; ++k) {
      const int32_t i = min(base + k * kWave + lane, L_cap - 1);
      o[k] = leaf_origin[i];
      bx[k] = leaf_box[i];
      inr[k] = leaf_inrun[i];
    }
  }
  if (L > L_cap || L < 0) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(flags, 2);
    L = L < 0 ? 0 : L_cap;
  }
  if (blockIdx.x != 0 && (int32_t)blockIdx.x * kFinSlice >= L) return;  // uniform per block
  const int32_t np = (L + (1 << gs) - 1) >> gs;  // runs of 2^gs leaves
  int32_t total = 0;
  if (L > 0) {  // uniform; np >= 1
    // first leaves' in-run counts (a grid without leaves points at the next
    // grid's first leaf, or at L): issued once gf is in, ahead of the scan
    int32_t fi[kG];
#pragma unroll
    for (int k = 0; k < kG; ++k) fi[k] = leaf_inrun[min(gf[k], L_cap - 1)];
    // run offsets
    int32_t rv[kR];
    int32_t sum = 0;
#pragma unroll
    for (int k = 0; k < kR; ++k) {
      rv[k] = tid * kR + k < np ? (int32_t)pv[k] : 0;
      sum += rv[k];
    }
    for (int g = tid; g < B; g += kFinThreads) {
      for (int a = 0; a < 3; ++a) {
        s_box[a][g] = INT32_MAX;
        s_box[3 + a][g] = INT32_MIN;
      }
    }
    int32_t ex = block_excl_scan<int32_t, kFinThreads>(sum, s_wave, total);
#pragma unroll
    for (int k = 0; k < kR; ++k) {
      s_part[tid * kR + k] = ex;
      ex += rv[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kG; ++k) {
      const int g = tid * kG + k;
      if (g < B) s_gvb[g] = gf[k] < L ? s_part[gf[k] >> gs] + fi[k] : total;
    }
    if (tid == 0) s_gvb[B] = total;
    __syncthreads();
    // leaf offsets and boxes: lane owns leaves base + k * 64 + lane
    int g = -1;
    int bv[6] = {INT32_MAX, INT32_MAX, INT32_MAX, INT32_MIN, INT32_MIN, INT32_MIN};
#pragma unroll
    for (int k = 0; k < kFinPer; ++k) {
      const int32_t i = base + k * kWave + lane;
      const int gk = o[k].w;
      if (i >= L || gk < 0 || gk >= B) continue;
      leaf_offset[i] = (i64)(s_part[i >> gs] + inr[k] - s_gvb[gk]);
      if (bx[k] == kEmptyBox) continue;
      if (gk != g) {
        if (g >= 0) box_fold_lds(s_box, g, bv);
        g = gk;
        for (int a = 0; a < 3; ++a) {
          bv[a] = INT32_MAX;
          bv[3 + a] = INT32_MIN;
        }
      }
      bv[0] = min(bv[0], o[k].x + (int)(bx[k] & 7));
      bv[3] = max(bv[3], o[k].x + (int)((bx[k] >> 3) & 7));
      bv[1] = min(bv[1], o[k].y + (int)((bx[k] >> 6) & 7));
      bv[4] = max(bv[4], o[k].y + (int)((bx[k] >> 9) & 7));
      bv[2] = min(bv[2], o[k].z + (int)((bx[k] >> 12) & 7));
      bv[5] = max(bv[5], o[k].z + (int)((bx[k] >> 15) & 7));
    }
    const bool act = g >= 0;
    const u64 am = __ballot(act);
    if (am) {  // uniform per wave
      const int first = __builtin_ctzll(am);
      const int g0 = __shfl(g, first, kWave);
      if (__ballot(act && g != g0) == 0) {  // one grid in every active lane: reduce, then one lane folds
        int r[6];
#pragma unroll
        for (int a = 0; a < 3; ++a) {
          r[a] = wave_min_i32(bv[a]);
          r[3 + a] = wave_max_i32(bv[3 + a]);
        }
        if (lane == first) box_fold_lds(s_box, g0, r);
      } else if (act) {
        box_fold_lds(s_box, g, bv);
      }
    }
    __syncthreads();
    for (int gg = tid; gg < B; gg += kFinThreads) {
      if (s_box[0][gg] == INT32_MAX) continue;  // no voxel of grid gg in this slice
      for (int a = 0; a < 3; ++a) {
        atomicMin(&hdr[gg].bbox_min[a], s_box[a][gg]);
        atomicMax(&hdr[gg].bbox_max[a], s_box[3 + a][gg]);
      }
    }
  } else {
    for (int g = tid; g <= B; g += kFinThreads) s_gvb[g] = 0;
    __syncthreads();
  }
  if (blockIdx.x != 0) return;
  // thread 0 made any flag update of this kernel itself; the writers ran before it
  if (tid < 4) status[tid] = tid == 0 ? *flags : 0;
#pragma unroll
  for (int k = 0; k < kG; ++k) {  // B <= kFinSmallGrids = kG * kFinThreads
    const int gg = tid + k * kFinThreads;
    if (gg >= B) break;
    tc_grid_header* h = hdr + gg;
    h->grid_index = gg;
    h->grid_count = B;
    h->upper_count = hv[k][0];
    h->lower_count = hv[k][1];
    h->leaf_count = hv[k][2];
    h->upper_begin = hv[k][3];
    h->lower_begin = hv[k][4];
    h->leaf_begin = hv[k][5];
    h->voxel_begin = s_gvb[gg];
    h->voxel_count = s_gvb[gg + 1] - s_gvb[gg];
    if (L == 0) {  // no leaves: no node writer ran and no box was folded
      for (int a = 0; a < 3; ++a) {
        h->bbox_min[a] = INT32_MAX;
        h->bbox_max[a] = INT32_MIN;
      }
    }
    h->reserved[0] = 0;
    h->reserved[1] = 0;
  }
  if (!host_words) return;
  // the host mirror: every header's node and voxel counts and begins (its box,
  // folded by every workgroup, is left out) and the status word after them
  tc_grid_header* hh = reinterpret_cast<tc_grid_header*>(host_words);
#pragma unroll
  for (int k = 0; k < kG; ++k) {
    const int gg = tid + k * kFinThreads;
    if (gg >= B) break;
    int32_t* w = reinterpret_cast<int32_t*>(hh + gg);
    w[0] = gg;
    w[1] = B;
#pragma unroll
    for (int f = 0; f < 6; ++f) w[2 + f] = hv[k][f];
    int64_t* v = reinterpret_cast<int64_t*>(&hh[gg].voxel_count);
    v[0] = s_gvb[gg + 1] - s_gvb[gg];
    v[1] = s_gvb[gg];
  }
  if (tid < 4) host_words[(sizeof(tc_grid_header) * (size_t)B) / 4 + tid] = tid == 0 ? *flags : 0;
}

__global__ void __launch_bounds__(kFinThreads) k_finalize_small(const int4* leaf_origin, const int32_t* leaf_inrun,
                                                                const uint32_t* leaf_box, const i64* vox_part,
                                                                int32_t gs, const int32_t* grid_info,
                                                                i64* leaf_offset, int32_t B, const int32_t* d_L,
                                                                int32_t L_cap, tc_grid_header* hdr,
                                                                int32_t* flags, int32_t* status,
                                                                int32_t* host_words) {
  finalize_small_body(leaf_origin, leaf_inrun, leaf_box, vox_part, gs, grid_info, leaf_offset, B, d_L, L_cap, hdr,
                      flags, status, host_words);
}

// Large batches: the leaf producer left one voxel sum per run of `gran` leaves
// (vox_part). One workgroup scans those sums, sets up the bbox accumulators and
// derives every grid's voxel begin (its first leaf's run offset plus the leaves
// before it in that run; gvb[B] = total); then every leaf's offset comes from its
// block's run offset plus a block scan, with no pass over all leaves just to scan.
constexpr int kPartThreads = 1024;
constexpr int kPartItems = 8;

__global__ void __launch_bounds__(kPartThreads) k_vox_partials(i64* vox_part, i64 np, const int32_t* leaf_inrun,
                                                               i64 gran, const int32_t* grid_info, int32_t B, i64 L,
                                                               int32_t* bbox, int32_t R, i64* gvb) {
  __shared__ i64 s_wave[kPartThreads / kWave];
  i64 carry = 0;
  for (i64 c = 0; c < np; c += (i64)kPartThreads * kPartItems) {
    i64 v[kPartItems];
    i64 sum = 0;
    const i64 base = c + (i64)threadIdx.x * kPartItems;
#pragma unroll
    for (int k = 0; k < kPartItems; ++k) v[k] = vox_part[min(base + k, np - 1)];  // clamped: all in flight
#pragma unroll
    for (int k = 0; k < kPartItems; ++k) {
      if (base + k >= np) v[k] = 0;
      sum += v[k];
    }
    i64 total;
    i64 ex = block_excl_scan<i64, kPartThreads>(sum, s_wave, total) + carry;
#pragma unroll
    for (int k = 0; k < kPartItems; ++k) {
      if (base + k < np) vox_part[base + k] = ex;
      ex += v[k];
    }
    carry += total;
  }
  for (i64 k = threadIdx.x; k < 3 * (i64)R * B; k += kPartThreads) {
    bbox[k] = INT32_MAX;
    bbox[3 * (i64)R * B + k] = INT32_MIN;
  }
  __syncthreads();  // the scanned runs are read below (by this workgroup only)
  // a grid's voxel begin: its first leaf's run offset plus that leaf's in-run prefix
  for (int32_t g = threadIdx.x; g <= B; g += kPartThreads) {
    const i64 f = g < B ? grid_info[g * 6 + 5] : L;
    gvb[g] = f < L ? vox_part[f >> __builtin_ctzll((u64)gran)] + leaf_inrun[f] : carry;
  }
}

// Per leaf: offset inside its grid and the per-grid bbox (as k_leaf_offsets_bbox).
__global__ void __launch_bounds__(256) k_leaf_offsets_runs(const int4* leaf_origin, const int32_t* leaf_inrun,
                                                           const uint32_t* leaf_box, const i64* vox_part, i64 gran,
                                                           const i64* gvb, i64* leaf_offset, int32_t* bbox,
                                                           int32_t B, int32_t R, i64 n_leaf) {
  const i64 i = (i64)blockIdx.x * 256 + threadIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const i64 ex = i < n_leaf ? vox_part[i >> __builtin_ctzll((u64)gran)] + leaf_inrun[i] : 0;  // batch-global voxel index of the leaf
  int g = -1;
  int bv[6] = {INT32_MAX, INT32_MAX, INT32_MAX, INT32_MIN, INT32_MIN, INT32_MIN};
  if (i < n_leaf) {
    const int4 o = leaf_origin[i];
    const uint32_t bx = leaf_box[i];
    if (o.w >= 0 && o.w < B) {
      leaf_offset[i] = ex - gvb[o.w];
      if (bx != kEmptyBox) {
        g = o.w;
        bv[0] = o.x + (int)(bx & 7);
        bv[3] = o.x + (int)((bx >> 3) & 7);
        bv[1] = o.y + (int)((bx >> 6) & 7);
        bv[4] = o.y + (int)((bx >> 9) & 7);
        bv[2] = o.z + (int)((bx >> 12) & 7);
        bv[5] = o.z + (int)((bx >> 15) & 7);
      }
    }
  }
  const bool active = g >= 0;
  const u64 act = __ballot(active);
  if (!act) return;  // uniform per wave; no barrier follows
  const int rep = (int)(blockIdx.x % (unsigned)R);
  const int first = __builtin_ctzll(act);
  const int g0 = __shfl(g, first, kWave);
  if (__ballot(active && g != g0) == 0) {
    int r[6];
#pragma unroll
    for (int a = 0; a < 3; ++a) {
      r[a] = wave_min_i32(bv[a]);
      r[3 + a] = wave_max_i32(bv[3 + a]);
    }
    if (lane == first) box_flush(bbox, B, R, rep, g0, r);
  } else if (active) {
    box_flush(bbox, B, R, rep, g, bv);
  }
}

// One wave per grid: lanes fold the bbox replicas, lane 0 writes the header.
__global__ void __launch_bounds__(256) k_write_headers_gvb(const int32_t* grid_info, const i64* gvb,
                                                           const int32_t* bbox, int32_t B, int32_t R,
                                                           tc_grid_header* hdr, const int32_t* flags,
                                                           int32_t* status) {
  const i64 g = (i64)blockIdx.x * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (blockIdx.x == 0 && threadIdx.x < 4) status[threadIdx.x] = threadIdx.x == 0 ? *flags : 0;
  if (g >= B) return;  // uniform per wave
  int v[6] = {INT32_MAX, INT32_MAX, INT32_MAX, INT32_MIN, INT32_MIN, INT32_MIN};
  for (int r = lane; r < R; r += kWave) {
#pragma unroll
    for (int a = 0; a < 3; ++a) {
      v[a] = min(v[a], bbox[((i64)a * R + r) * B + g]);
      v[3 + a] = max(v[3 + a], bbox[((i64)(3 + a) * R + r) * B + g]);
    }
  }
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    v[a] = wave_min_i32(v[a]);
    v[3 + a] = wave_max_i32(v[3 + a]);
  }
  if (lane != 0) return;
  const int32_t* gi = grid_info + g * 6;
  tc_grid_header h;
  h.grid_index = (int32_t)g;
  h.grid_count = B;
  h.upper_count = gi[0];
  h.lower_count = gi[1];
  h.leaf_count = gi[2];
  h.upper_begin = gi[3];
  h.lower_begin = gi[4];
  h.leaf_begin = gi[5];
  h.voxel_begin = gvb[g];
  h.voxel_count = gvb[g + 1] - gvb[g];
  for (int a = 0; a < 3; ++a) {
    h.bbox_min[a] = v[a];
    h.bbox_max[a] = v[3 + a];
  }
  h.reserved[0] = 0;
  h.reserved[1] = 0;
  hdr[g] = h;
}

bool finalize_small_fits(i64 L, int32_t B, i64 gran) {
  return L <= kFinSmallLeaves && B <= kFinSmallGrids && ceil_div(L, gran) <= kFinRuns;
}

void tree_finalize_leaves(const GridView& out, const uint32_t* leaf_box, const int32_t* leaf_inrun, i64* vox_part,
                          i64 gran, i64* gvb, int32_t* bbox_accum, const int32_t* grid_info, int32_t* flags,
                          const int32_t* d_L, hipStream_t s, int32_t* host_words) {
  if (host_words && !finalize_small_fits(out.n_leaf, out.B, gran))
    throw Error(TC_ERR_INTERNAL, "finalize: a host mirror needs the one-launch finalize");
  const i64 L = out.n_leaf;  // the leaf count, or (d_L given) a capacity with the count at d_L
  const int32_t B = out.B;
  if (gran <= 0 || (gran & (gran - 1)) != 0) throw Error(TC_ERR_INTERNAL, "finalize: run length not a power of two");
  if (finalize_small_fits(L, B, gran)) {
    launch("k_finalize_small", k_finalize_small, std::max<i64>(1, ceil_div(L, kFinSlice)), kFinThreads, s,
           (const int4*)out.leaf_origin, leaf_inrun, leaf_box, (const i64*)vox_part,
           (int32_t)__builtin_ctzll((u64)gran), grid_info, out.leaf_offset, B, d_L, (int32_t)L, out.headers,
           flags, out.status, host_words);
    return;
  }
  // the wide path runs on exact counts only (its launches are sized by them)
  const int32_t R = bbox_replicas(B);
  launch("k_vox_partials", k_vox_partials, 1, kPartThreads, s, vox_part, ceil_div(L, gran), leaf_inrun, gran,
         grid_info, B, L, bbox_accum, R, gvb);
  launch("k_leaf_offsets_bbox", k_leaf_offsets_runs, ceil_div(L, 256), 256, s, (const int4*)out.leaf_origin,
         leaf_inrun, leaf_box, (const i64*)vox_part, gran, (const i64*)gvb, out.leaf_offset, bbox_accum, B, R, L);
  launch("k_write_headers", k_write_headers_gvb, ceil_div((i64)B, 4), 256, s, grid_info, (const i64*)gvb,
         (const int32_t*)bbox_accum, B, R, out.headers, flags, out.status);
}

// ------------------------------------------------------------------ enumeration
// One wave walks `lpw` (1..8) consecutive leaves. Their masks, prefix words,
// origins and voxel offsets are loaded once, up front, while the block stages
// the grids' voxel begins in LDS (so no load waits on a leaf's grid index); many
// leaves per wave amortise the load latency on large batches, one leaf per wave
// keeps small batches wide. For each leaf, lane r owns row r = x*8 + y (byte y
// of word x, at most 8 voxels along z). The row's first voxel is the leaf's
// prefix field for the words before x plus the set bits of word x before byte
// y, so no cross-lane scan is needed; lanes expand their rows into LDS in bit
// order, and the wave streams the leaf's rows out with 16-byte stores (the LDS
// image is shifted so that its 16-byte chunks line up with the destination's).
// Launches below eight leaves per wave (up to 256K leaves) make them
// non-temporal: their output then leaves few dirty lines behind at the kernel's
// end (measured faster there, and slower on the largest launches). The wave index is
// made uniform, so the per-leaf values of the loop come from lane reads.
constexpr int kEnumMaxLeaves = 8;
constexpr int kEnumLdsGrids = 256;  // up to this many grids, voxel begins come from LDS

// Kernel argument of k_enumerate_many: up to kEnumMany batches.
constexpr int kEnumMany = 8;
struct EnumBatch {
  const tc_grid_header* hdr;
  const int4* leaf_origin;
  const u64* leaf_mask;
  const u64* leaf_prefix;
  const i64* leaf_offset;
  int32_t* ijk;
  i64 n_leaf;
  int32_t B;
  int32_t vec_ok;
};
struct EnumBatches {
  EnumBatch b[kEnumMany];
  i64 block_begin[kEnumMany];
  int32_t n;
  int32_t lpw;
};

typedef int v4i32 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i64 readlane64(i64 v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((u64)v >> 32), l);
  return (i64)(((u64)hi << 32) | lo);
}

// One block's share (block `blk` of the batch's launch shape) of k_enumerate.
template <bool NT>
__device__ __forceinline__ void enumerate_block(const tc_grid_header* hdr, const int4* leaf_origin,
                                                const u64* leaf_mask, const u64* leaf_prefix,
                                                const i64* leaf_offset, int32_t* ijk, i64 n_leaf, int32_t B,
                                                int lpw, int vec_ok, i64 blk,
                                                int32_t (*s_rows)[3 * 512 + 4], i64* s_vb) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  const i64 l0 = (blk * 4 + w) * lpw;
  const int nl = (int)max((i64)0, min((i64)lpw, n_leaf - l0));
  const int jl = lane >> 3;
  const u64 myword = jl < nl ? leaf_mask[(l0 + jl) * 8 + (lane & 7)] : 0ull;
  int4 myo = make_int4(0, 0, 0, 0);
  i64 myoff = 0;
  u64 mypre = 0;
  if (lane < nl) {
    myo = leaf_origin[l0 + lane];
    myoff = leaf_offset[l0 + lane];
    mypre = leaf_prefix[l0 + lane];
  }
  const bool lds_vb = B <= kEnumLdsGrids;  // uniform
  if (lds_vb) {
    for (int g = threadIdx.x; g < B; g += 256) s_vb[g] = hdr[g].voxel_begin;
    __syncthreads();
  }
  if (nl == 0) return;  // uniform per wave; no block barrier below
  i64 mybase = 0;
  if (lane < nl) mybase = (lds_vb ? s_vb[myo.w] : hdr[myo.w].voxel_begin) + myoff;
  int32_t* rows = s_rows[w];
  const int x = lane >> 3, y = lane & 7;
  const u64 below = (1ull << (8 * y)) - 1;  // the bits of word x before row y
  for (int j = 0; j < nl; ++j) {
    const u64 word = __shfl(myword, j * 8 + x, kWave);
    const int ox = __builtin_amdgcn_readlane(myo.x, j), oy = __builtin_amdgcn_readlane(myo.y, j),
              oz = __builtin_amdgcn_readlane(myo.z, j);
    const i64 base = readlane64(mybase, j);
    const u64 pre = (u64)readlane64((i64)mypre, j);
    const uint32_t row = (uint32_t)(word >> (8 * y)) & 0xffu;
    // voxels before this row: in the words before x (prefix field x - 1), then in word x
    const int pw = x == 0 ? 0 : (int)((pre >> (9 * (x - 1))) & 511u);
    const int ex = pw + popc64(word & below);
    const int total = __builtin_amdgcn_readlane(ex + __popc(row), kWave - 1);  // lane 63: the last row
    const int a = vec_ok ? (int)((base * 3) & 3) : 0;
    int at = a + 3 * ex;
    const int X = ox + x, Y = oy + y;
    uint32_t rest = row;
    while (rest) {
      const int z = __builtin_ctz(rest);
      rows[at + 0] = X;
      rows[at + 1] = Y;
      rows[at + 2] = oz + z;
      rest &= rest - 1;
      at += 3;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int n = a + 3 * total;
    int32_t* dst = ijk + base * 3 - a;  // 16-byte aligned when vec_ok
    if (vec_ok) {
      v4i32* dst4 = reinterpret_cast<v4i32*>(dst);
      const v4i32* src4 = reinterpret_cast<const v4i32*>(rows);
      const int nq = (n + 3) >> 2;
      for (int q0 = 0; q0 < nq; q0 += 2 * kWave) {
        v4i32 v[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int q = q0 + u * kWave + lane;
          if (q < nq) v[u] = src4[q];
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int q = q0 + u * kWave + lane;
          const int e0 = q * 4;
          if (q >= nq) continue;
          if (e0 >= a && e0 + 4 <= n) {
            if constexpr (NT) __builtin_nontemporal_store(v[u], dst4 + q);
            else dst4[q] = v[u];
          } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              if (e0 + t >= a && e0 + t < n) {
                if constexpr (NT) __builtin_nontemporal_store(v[u][t], dst + e0 + t);
                else dst[e0 + t] = v[u][t];
              }
            }
          }
        }
      }
    } else {
      for (int e = lane; e < n; e += kWave) dst[e] = rows[e];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

template <bool NT>
__global__ void __launch_bounds__(256) k_enumerate(const tc_grid_header* hdr, const int4* leaf_origin,
                                                   const u64* leaf_mask, const u64* leaf_prefix,
                                                   const i64* leaf_offset, int32_t* ijk, i64 n_leaf, int32_t B,
                                                   int lpw, int vec_ok) {
  __shared__ __align__(16) int32_t s_rows[4][3 * 512 + 4];
  __shared__ i64 s_vb[kEnumLdsGrids];  // grids' voxel begins, loaded beside the leaves
  enumerate_block<NT>(hdr, leaf_origin, leaf_mask, leaf_prefix, leaf_offset, ijk, n_leaf, B, lpw, vec_ok,
                      blockIdx.x, s_rows, s_vb);
}

// Several batches in one launch: the blocks of batch j follow those of batch
// j - 1 (block_begin, by value); every block finds its batch among at most
// kEnumMany and runs that batch's share. One launch fills the chip where a
// small batch alone would not, and saves the launches.
template <bool NT>
__global__ void __launch_bounds__(256) k_enumerate_many(EnumBatches eb) {
  __shared__ __align__(16) int32_t s_rows[4][3 * 512 + 4];
  __shared__ i64 s_vb[kEnumLdsGrids];
  int j = 0;
#pragma unroll
  for (int q = 1; q < kEnumMany; ++q) j += q < eb.n && (i64)blockIdx.x >= eb.block_begin[q] ? 1 : 0;
  const EnumBatch& b = eb.b[j];
  enumerate_block<NT>(b.hdr, b.leaf_origin, b.leaf_mask, b.leaf_prefix, b.leaf_offset, b.ijk, b.n_leaf, b.B,
                      eb.lpw, b.vec_ok, (i64)blockIdx.x - eb.block_begin[j], s_rows, s_vb);
}

// one leaf per wave while the waves fit in one round of the chip (about 6k
// resident at this LDS use), then two, then eight on large batches
static int enumerate_lpw(i64 n_leaf) { return n_leaf >= 256 * 1024 ? kEnumMaxLeaves : (n_leaf >= 6 * 1024 ? 2 : 1); }

void tree_enumerate(const GridView& v, int32_t* ijk, hipStream_t s) {
  const int vec_ok = (reinterpret_cast<uintptr_t>(ijk) & 15) == 0 ? 1 : 0;
  const int lpw = enumerate_lpw(v.n_leaf);
  launch("k_enumerate", lpw < kEnumMaxLeaves ? k_enumerate<true> : k_enumerate<false>, ceil_div((i64)v.n_leaf, 4 * lpw), 256, s,
         (const tc_grid_header*)v.headers, (const int4*)v.leaf_origin, (const u64*)v.leaf_mask,
         (const u64*)v.leaf_prefix, (const i64*)v.leaf_offset, ijk, (i64)v.n_leaf, v.B, lpw, vec_ok);
}

void tree_enumerate_many(const GridView* v, int32_t* const* ijk, int n, hipStream_t s) {
  for (int j0 = 0; j0 < n; j0 += kEnumMany) {
    const int m = std::min(kEnumMany, n - j0);
    i64 leaves = 0;
    for (int j = 0; j < m; ++j) leaves += v[j0 + j].n_leaf;
    EnumBatches eb{};
    eb.n = m;
    eb.lpw = enumerate_lpw(leaves);  // one launch shape for the whole launch
    i64 blocks = 0;
    for (int j = 0; j < m; ++j) {
      const GridView& g = v[j0 + j];
      EnumBatch& b = eb.b[j];
      b.hdr = g.headers;
      b.leaf_origin = g.leaf_origin;
      b.leaf_mask = g.leaf_mask;
      b.leaf_prefix = g.leaf_prefix;
      b.leaf_offset = g.leaf_offset;
      b.ijk = ijk[j0 + j];
      b.n_leaf = g.n_leaf;
      b.B = g.B;
      b.vec_ok = (reinterpret_cast<uintptr_t>(b.ijk) & 15) == 0 ? 1 : 0;
      eb.block_begin[j] = blocks;
      blocks += ceil_div((i64)g.n_leaf, 4 * eb.lpw);
    }
    for (int j = m; j < kEnumMany; ++j) eb.block_begin[j] = blocks;
    launch("k_enumerate", eb.lpw < kEnumMaxLeaves ? k_enumerate_many<true> : k_enumerate_many<false>, blocks, 256,
           s, eb);
  }
}

}  // namespace tc
