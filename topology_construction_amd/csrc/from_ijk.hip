// Grid batch from int32 voxel rows: the ijk emission front-end (PR page,
// Measurements: the follow-up ijk front-end on the same back-end; Test plan:
// expected topologies are built from ijk).
//
// The rows are read once. They are cut into chunks of kRecChunk consecutive
// rows, and every chunk is folded into leaf-word records: rows that fall into
// the same 64-bit word of the same leaf mask (same grid, same x, same leaf y and
// z) OR their voxel bits together, first along each lane's own rows, then
// through a hash table in LDS. A record keeps a representative position (x
// exact, y and z rounded down to their leaf) and its root tile, from which every
// coarser level follows as from any voxel of the word. Root tiles are
// deduplicated as the records are written, through a global open-addressing
// table whose slots hold a representative row; the few unique tiles are then
// sorted, and the levels below them are assembled from the records with the
// bitmap-rank tree assembly of the topology pass. Two readbacks size the
// scratch arrays (records, tiles and lower keys; node counts).
#include <algorithm>
#include <cstring>
#include <memory>

#include "device.hpp"
#include "internal.hpp"

namespace tc {

// Member of row i: the last g with offsets[g] <= i (binary search).
__device__ __forceinline__ int32_t member_of(const i64* offsets, int32_t B, i64 i) {
  int32_t lo = 0, hi = B - 1;
  while (lo < hi) {
    const int32_t mid = lo + (hi - lo + 1) / 2;
    if (offsets[mid] <= i) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Control words of the record pass, read back together: [0] unused, [1] tiles
// claimed, [2] flags, [3] tile collection counter (after the readback), [4]
// lower keys, [5] records.
constexpr int kCtlWords = 8;
constexpr int32_t kRetryFlag = 8;  // the tile table filled past half: the pass runs again with a larger one
constexpr i64 kTileTableFirst = 1 << 16;

// ------------------------------------------------------------------ LDS word table
// Candidate-lower and tile-lower words: a block ORs the bits of its items into
// an LDS hash table keyed by word address (LDS compare-and-swap claims a key,
// LDS OR merges the bits), then ORs each distinct word once, reading the global
// word first and skipping the OR when its bits are already set. The global ORs
// are device-scope atomics, which on this multi-XCD part resolve past the
// per-XCD L2 and serialize per address: merging first keeps them few.
constexpr int kBlockTable = 2048;  // entries; at most kPerBlock keys per fill, so probes stay short

__device__ __forceinline__ void table_clear(unsigned long long* key, unsigned long long* val) {
  for (int e = threadIdx.x; e < kBlockTable; e += 256) {
    key[e] = 0ull;
    val[e] = 0ull;
  }
}

// Every insert finds its key or a free entry within kBlockTable probes because
// the table holds at most kPerBlock keys.
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

// ORs the table's words into global memory and clears the entries (each thread
// the ones it read), ready for the next fill after a barrier.
__device__ __forceinline__ void table_flush_clear(unsigned long long* key, unsigned long long* val) {
  constexpr int kPer = kBlockTable / 256;
  unsigned long long k[kPer], v[kPer], cur[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    k[j] = key[threadIdx.x + 256 * j];
    v[j] = val[threadIdx.x + 256 * j];
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) cur[j] = k[j] ? *reinterpret_cast<const u64*>((uintptr_t)k[j]) : 0ull;
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (k[j] && (cur[j] & v[j]) != v[j]) atomicOr(reinterpret_cast<unsigned long long*>((uintptr_t)k[j]), v[j]);
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (k[j]) {
      key[threadIdx.x + 256 * j] = 0ull;
      val[threadIdx.x + 256 * j] = 0ull;
    }
}

// ------------------------------------------------------------------ tile table
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

// table[H] holds -1 or a row of the first record seen for a (grid, tile); the
// rows never change during the pass, so a slot is complete once claimed.
// Returns the slot of (g, tx, ty, tz), claiming one with row `e` if none holds
// it. Claims are counted in ctl[1]; past H/2 of them, or when no slot is found
// within H probes, the pass is flagged for a rerun with a larger table (-1).
__device__ __attribute__((noinline)) int32_t tile_slot(const int32_t* ijk, const i64* offsets, int32_t B, int32_t e,
                                                      int32_t g, int32_t tx, int32_t ty, int32_t tz, int32_t* table,
                                                      i64 H, int32_t* ctl) {
  i64 h = (i64)(tile_hash(g, tx, ty, tz) & (u64)(H - 1));
  for (i64 probe = 0; probe < H; ++probe) {
    // A claimed slot never changes, so a plain (possibly stale) read can only
    // miss a claim, which the compare-and-swap then returns. Device-scope reads
    // of one hot slot would all queue at its memory channel.
    int32_t r = table[h];
    if (r < 0) {
      const int32_t old = atomicCAS(&table[h], -1, e);
      if (old < 0) {
        const int32_t claimed = atomicAdd(&ctl[1], 1) + 1;
        if (2 * (i64)claimed > H) atomicOr(&ctl[2], kRetryFlag);
        return (int32_t)h;
      }
      r = old;
    }
    if ((ijk[(i64)r * 3] >> 12) == tx && (ijk[(i64)r * 3 + 1] >> 12) == ty && (ijk[(i64)r * 3 + 2] >> 12) == tz &&
        offsets[g] <= r && r < offsets[g + 1])
      return (int32_t)h;
    h = (h + 1) & (H - 1);
  }
  atomicOr(&ctl[2], kRetryFlag);
  return -1;
}

// ------------------------------------------------------------------ records
constexpr int kRecRows = 4;                // consecutive rows per lane
constexpr int kRecChunk = 256 * kRecRows;  // rows per chunk
constexpr int kRecTableBits = 11;
constexpr int kRecTable = 1 << kRecTableBits;  // LDS table entries
constexpr int32_t kRecSpan = 1 << 15;          // range of a packed-key field
constexpr u64 kRecEmpty = ~0ull;
constexpr int kRecBlocksPerCu = 3;  // workgroups of the record pass per compute unit (its LDS use)
// A chunk has at most kRecChunk keys, so a probe always ends at its key or a
// free entry.
static_assert(kRecTable >= kRecChunk, "the LDS table takes every key of a chunk");

// Records are stored by region: workgroup w of the record pass takes chunks
// [w * cpw, (w + 1) * cpw) and writes its records (and its lower keys) from
// slot w * cpw * kRecChunk on (the first row of its first chunk: a region holds
// at most one record per row); region_cnt[w] and region_lcnt[w] count them.
// Consumers take part (blockIdx.x mod split) of region (blockIdx.x / split), in
// steps of split * span items.
struct RegionPart {
  i64 base;     // first slot of the region
  int32_t cnt;  // items in the region
  int32_t first, step;
};
__device__ __forceinline__ RegionPart region_part(const int32_t* counts, i64 cpw, int split, int span) {
  const i64 w = blockIdx.x / split;
  RegionPart p;
  p.base = w * cpw * kRecChunk;
  p.cnt = counts[w];
  p.first = (int32_t)(blockIdx.x % split) * span;
  p.step = split * span;
  return p;
}

// First-level loads of the consumers do not wait for the region's count: they
// read slot min(base + j, last) (inside the arrays whatever j is) and the item
// is dropped afterwards when j is past the count.
__device__ __forceinline__ i64 clamp_slot(i64 slot, i64 last) { return slot < last ? slot : last; }

// Item v of this lane in a step of V items per lane: the wave's 64 V items are
// consecutive, slot v holding items 64 v + lane.
template <int V>
__device__ __forceinline__ int32_t step_item(int v) {
  return (int32_t)((threadIdx.x / kWave) * (kWave * V) + v * kWave + (threadIdx.x & (kWave - 1)));
}

// Chunk c: the grid of its first row (chunk_g[C] is the grid of the last row),
// and the tile slot of its first row, which most of its records share.
__global__ void __launch_bounds__(256) k_chunk_prep(const int32_t* ijk, const i64* offsets, int32_t B, i64 n,
                                                    i64 C, int32_t* chunk_g, int32_t* chunk_tslot, int32_t* table,
                                                    i64 H, int32_t* ctl) {
  const i64 c = (i64)blockIdx.x * 256 + threadIdx.x;
  if (c > C) return;
  if (c == C) {
    chunk_g[C] = member_of(offsets, B, n - 1);
    return;
  }
  const i64 row = c * kRecChunk;
  const int32_t g = member_of(offsets, B, row);
  chunk_g[c] = g;
  chunk_tslot[c] = tile_slot(ijk, offsets, B, (int32_t)row, g, ijk[row * 3] >> 12, ijk[row * 3 + 1] >> 12,
                             ijk[row * 3 + 2] >> 12, table, H, ctl);
}

// Key of a word relative to the chunk's first row: grid, x, leaf-y and leaf-z
// differences in 16-bit fields. The grid difference lies in [0, 2^15), so no
// key reaches kRecEmpty.
__device__ __forceinline__ u64 rec_pack(int32_t dg, int32_t dx, int32_t dy, int32_t dz) {
  return ((u64)(uint32_t)dg << 48) | ((u64)(uint16_t)dx << 32) | ((u64)(uint16_t)dy << 16) | (u64)(uint16_t)dz;
}

// |a - b| < 2^15 for any two int32 values, without 64-bit arithmetic: their
// high halves differ by at most one, so the wrapped difference is exact.
__device__ __forceinline__ bool near15(int32_t a, int32_t b) {
  const int32_t dh = (a >> 16) - (b >> 16);
  const int32_t d = (int32_t)((uint32_t)a - (uint32_t)b);
  return dh >= -1 && dh <= 1 && d >= -kRecSpan && d < kRecSpan;
}

// Lower key of a record: its tile slot and its lower's bit in the tile's
// 32^3 lower mask.
__device__ __forceinline__ i64 lower_key(int32_t slot, int32_t x, int32_t y, int32_t z) {
  return ((i64)slot << 15) | ((((x >> 7) & 31) * 32 + ((y >> 7) & 31)) * 32 + ((z >> 7) & 31));
}

// Lists lower key lk once per chunk: an LDS set of kLowSet keys filters
// repeats; a key that finds the set full is listed again (the marking ORs
// repeats away). At most one listing per record.
constexpr int kLowSet = 256;
__device__ __forceinline__ void lower_add(i64 lk, u64* s_low, int32_t* s_lcnt, i64* low_out) {
  unsigned h = ((uint32_t)lk * 0x9e3779b1u ^ (uint32_t)((u64)lk >> 32) * 0x85ebca6bu) >> 24;
  u64 prev;
  int probe = 0;
#pragma unroll 1
  do {  // one exit: the key's entry, a free entry, or a full set
    prev = atomicCAS((unsigned long long*)&s_low[h], (unsigned long long)kRecEmpty, (unsigned long long)lk);
    h = (h + 1) & (kLowSet - 1);
  } while (prev != kRecEmpty && prev != (u64)lk && ++probe < kLowSet);
  if (prev != (u64)lk) low_out[atomicAdd(s_lcnt, 1)] = lk;
}

// Claims or finds `key` in the LDS table and ORs `bits` into its entry. The
// claiming lane takes the chunk's next record position (s_cnt), lists the
// entry there and stores its representative row. The table holds at most
// kRecChunk keys, so a free entry is always found.
__device__ __forceinline__ void rec_insert(u64* s_key, u64* s_bits, int32_t* s_rep, int16_t* s_list, int32_t* s_cnt,
                                           u64 key, u64 bits, int32_t rep, int32_t* flags) {
  unsigned h = ((uint32_t)key * 0x9e3779b1u ^ (uint32_t)(key >> 32) * 0x85ebca6bu) >> (32 - kRecTableBits);
  u64 prev;
  int probe = 0;
#pragma unroll 1
  do {  // one exit: the key's entry or a free one (always found: a chunk has at most kRecChunk keys)
    prev = atomicCAS((unsigned long long*)&s_key[h], (unsigned long long)kRecEmpty, (unsigned long long)key);
    if (prev == kRecEmpty || prev == key) break;
    h = (h + 1) & (kRecTable - 1);
  } while (++probe < kRecTable);
  if (prev != kRecEmpty && prev != key) {  // consistency guard
    atomicOr(flags, kFlagInternal);
    return;
  }
  if (prev == kRecEmpty) {
    s_rep[h] = rep;
    s_list[atomicAdd(s_cnt, 1)] = (int16_t)h;
  }
  atomicOr((unsigned long long*)&s_bits[h], (unsigned long long)bits);
}

// The record pass. One persistent workgroup per region; it takes the region's
// chunks in turn, loading the next chunk's rows while it merges the current
// one. Lane l holds rows l * kRecRows .. + kRecRows - 1 of the chunk and merges
// its runs of rows in one word. When every row of a wave lies within 2^15 of
// the chunk's first row in grid, x, leaf y and leaf z (the common case: rows
// of a grid arrive roughly in order), its runs merge further through the LDS
// table keyed by packed words, whose entries become records; otherwise each of
// its runs is a record of its own. A record is written as (x, y and z rounded
// down to the leaf, tile slot) with its bits, and its lower key is listed once
// per chunk. No counter is shared between workgroups.
__global__ void __launch_bounds__(256) k_ijk_records(const int32_t* ijk, const i64* offsets, int32_t B, i64 n,
                                                     const int32_t* chunk_g, const int32_t* chunk_tslot, i64 C,
                                                     i64 cpw, int4* rec_cap, u64* bits_cap, i64* low_cap,
                                                     int32_t* region_cnt, int32_t* region_lcnt, int32_t* table,
                                                     i64 H, int32_t* ctl) {
  __shared__ u64 s_key[kRecTable];
  __shared__ u64 s_bits[kRecTable];
  __shared__ int32_t s_rep[kRecTable];
  __shared__ u64 s_low[kLowSet];
  __shared__ int16_t s_list[kRecChunk];
  __shared__ int32_t s_cnt, s_lcnt;
  static_assert(kLowSet == 256, "one set entry per thread");
  const i64 w = blockIdx.x;
  const i64 c0 = w * cpw, c1 = min(C, c0 + cpw);
  const i64 rbase = c0 * kRecChunk;
  for (int e = threadIdx.x; e < kRecTable; e += 256) {
    s_key[e] = kRecEmpty;
    s_bits[e] = 0ull;
  }
  if (threadIdx.x == 0) {
    s_cnt = 0;
    s_lcnt = 0;
  }
  i64 out = rbase;  // next record slot of the region (uniform)
  int32_t nx[kRecRows], ny[kRecRows], nz[kRecRows];  // the next chunk's rows
  int32_t ngA = 0, ngB = 0, nts = 0, nx0 = 0, ny0 = 0, nz0 = 0;  // and its grid range, tile slot and first row
  auto load_rows = [&](i64 c) {
    ngA = chunk_g[c];
    ngB = chunk_g[c + 1];
    nts = chunk_tslot[c];
    nx0 = ijk[c * kRecChunk * 3];
    ny0 = ijk[c * kRecChunk * 3 + 1];
    nz0 = ijk[c * kRecChunk * 3 + 2];
    const i64 i0 = c * kRecChunk + (i64)threadIdx.x * kRecRows;
    if (c * kRecChunk + kRecChunk <= n) {  // uniform: a whole chunk, 12 * kRecRows contiguous bytes per lane
      const int32_t* p = ijk + i0 * 3;
#pragma unroll
      for (int r = 0; r < kRecRows; ++r) {
        nx[r] = p[3 * r];
        ny[r] = p[3 * r + 1];
        nz[r] = p[3 * r + 2];
      }
    } else {
#pragma unroll
      for (int r = 0; r < kRecRows; ++r) {
        const bool in = i0 + r < n;
        nx[r] = in ? ijk[(i0 + r) * 3] : 0;
        ny[r] = in ? ijk[(i0 + r) * 3 + 1] : 0;
        nz[r] = in ? ijk[(i0 + r) * 3 + 2] : 0;
      }
    }
  };
  if (c0 < c1) load_rows(c0);
  for (i64 c = c0; c < c1; ++c) {
    s_low[threadIdx.x] = kRecEmpty;
    int32_t x[kRecRows], y[kRecRows], z[kRecRows], g[kRecRows];
#pragma unroll
    for (int r = 0; r < kRecRows; ++r) {
      x[r] = nx[r];
      y[r] = ny[r];
      z[r] = nz[r];
    }
    const int32_t gA = ngA, gB = ngB, ts0 = nts, x0 = nx0, y0 = ny0, z0 = nz0;
    if (c + 1 < c1) load_rows(c + 1);
    const i64 base = c * kRecChunk;
    const i64 i0 = base + (i64)threadIdx.x * kRecRows;
    bool in[kRecRows];
#pragma unroll
    for (int r = 0; r < kRecRows; ++r) in[r] = i0 + r < n;
    const int32_t yb0 = y0 >> 3, zb0 = z0 >> 3;
    if (gA == gB) {  // uniform: the chunk lies in one grid
#pragma unroll
      for (int r = 0; r < kRecRows; ++r) g[r] = gA;
    } else {  // a search for the lane's first row, then steps over member ends
      int32_t gi = in[0] ? member_of(offsets, B, i0) : 0;
#pragma unroll
      for (int r = 0; r < kRecRows; ++r) {
        if (in[r])
          while (gi + 1 < B && offsets[gi + 1] <= i0 + r) ++gi;
        g[r] = gi;
      }
    }
    // packed keys; a row heads a run unless it lies in the previous row's word
    bool ok = true, head[kRecRows];
    u64 key[kRecRows], rb[kRecRows];
#pragma unroll
    for (int r = 0; r < kRecRows; ++r) {
      const int32_t dg = g[r] - gA, dy = (y[r] >> 3) - yb0, dz = (z[r] >> 3) - zb0;
      if (in[r])
        ok = ok && dg >= 0 && dg < kRecSpan && near15(x[r], x0) && dy >= -kRecSpan && dy < kRecSpan &&
             dz >= -kRecSpan && dz < kRecSpan;
      key[r] = rec_pack(dg, (int32_t)((uint32_t)x[r] - (uint32_t)x0), dy, dz);
    }
    const bool packed = __all(ok);  // uniform per wave
#pragma unroll
    for (int r = 0; r < kRecRows; ++r) {
      const bool cont = r > 0 && in[r] &&
                        (packed ? key[r] == key[r - 1]
                                : (g[r] == g[r - 1] && x[r] == x[r - 1] && (y[r] >> 3) == (y[r - 1] >> 3) &&
                                   (z[r] >> 3) == (z[r - 1] >> 3)));
      head[r] = in[r] && !cont;
    }
    {
      u64 acc = 0;
#pragma unroll
      for (int r = kRecRows - 1; r >= 0; --r) {
        if (in[r]) acc |= 1ull << (((y[r] & 7) << 3) | (z[r] & 7));
        rb[r] = head[r] ? acc : 0ull;
        if (head[r]) acc = 0;
      }
    }
    __syncthreads();  // the previous chunk's flush is over: list, counters and set are free
    if (packed) {
#pragma unroll
      for (int r = 0; r < kRecRows; ++r)
        if (head[r]) rec_insert(s_key, s_bits, s_rep, s_list, &s_cnt, key[r], rb[r], (int32_t)(i0 + r), &ctl[2]);
    } else {  // each run is a record now; its list entry says so
#pragma unroll
      for (int r = 0; r < kRecRows; ++r) {
        if (!head[r]) continue;
        const int32_t pos = atomicAdd(&s_cnt, 1);
        s_list[pos] = -1;
        const int32_t yy = y[r] & ~7, zz = z[r] & ~7;
        const int32_t slot =
            tile_slot(ijk, offsets, B, (int32_t)(i0 + r), g[r], x[r] >> 12, yy >> 12, zz >> 12, table, H, ctl);
        rec_cap[out + pos] = make_int4(x[r], yy, zz, slot);
        bits_cap[out + pos] = rb[r];
        if (slot >= 0) lower_add(lower_key(slot, x[r], yy, zz), s_low, &s_lcnt, low_cap + rbase);
      }
    }
    __syncthreads();
    const int32_t total = s_cnt;
    const int32_t tx0 = x0 >> 12, ty0 = y0 >> 12, tz0 = z0 >> 12;
    for (int j = threadIdx.x; j < total; j += 256) {
      const int e = s_list[j];
      if (e < 0) continue;
      const u64 k = s_key[e];
      const int32_t dg = (int32_t)(k >> 48), dx = (int16_t)(uint16_t)(k >> 32), dy = (int16_t)(uint16_t)(k >> 16),
                    dz = (int16_t)(uint16_t)k;
      const int32_t gx = gA + dg, xx = (int32_t)((uint32_t)x0 + (uint32_t)dx),
                    yy = (int32_t)((uint32_t)(yb0 + dy) << 3), zz = (int32_t)((uint32_t)(zb0 + dz) << 3);
      const int32_t slot = (gx == gA && (xx >> 12) == tx0 && (yy >> 12) == ty0 && (zz >> 12) == tz0)
                               ? ts0
                               : tile_slot(ijk, offsets, B, s_rep[e], gx, xx >> 12, yy >> 12, zz >> 12, table, H, ctl);
      rec_cap[out + j] = make_int4(xx, yy, zz, slot);
      bits_cap[out + j] = s_bits[e];
      s_key[e] = kRecEmpty;
      s_bits[e] = 0ull;
      if (slot >= 0) lower_add(lower_key(slot, xx, yy, zz), s_low, &s_lcnt, low_cap + rbase);
    }
    out += total;
    __syncthreads();  // every thread has read s_cnt
    if (threadIdx.x == 0) s_cnt = 0;
  }
  __syncthreads();
  if (threadIdx.x == 0 && c0 < C) {
    const int32_t nrec = (int32_t)(out - rbase), nlow = s_lcnt;
    region_cnt[w] = nrec;
    region_lcnt[w] = nlow;
    atomicAdd(&ctl[5], nrec);
    atomicAdd(&ctl[4], nlow);
  }
}

// Unique tiles: every claimed slot of the tile table, in any order, with its
// sort key (the slot is the value).
__global__ void __launch_bounds__(256) k_tile_collect(const int32_t* table, i64 H, const int32_t* ijk,
                                                      const i64* offsets, int32_t B, int32_t nt, int32_t* counter,
                                                      Key128* keys, uint32_t* vals, int32_t* flags) {
  const i64 h = (i64)blockIdx.x * 256 + threadIdx.x;
  if (h >= H) return;
  const int32_t e = table[h];
  if (e < 0) return;
  const int32_t k = atomicAdd(counter, 1);
  if (k >= nt) {  // consistency guard: more claimed slots than claims
    atomicOr(flags, kFlagInternal);
    return;
  }
  const u64 g = (uint32_t)member_of(offsets, B, e);
  const u64 tx = (u64)((ijk[(i64)e * 3] >> 12) + kTileBias), ty = (u64)((ijk[(i64)e * 3 + 1] >> 12) + kTileBias),
            tz = (u64)((ijk[(i64)e * 3 + 2] >> 12) + kTileBias);
  keys[k] = Key128{((g & 15ull) << 60) | (tx << 40) | (ty << 20) | tz, g >> 4};
  vals[k] = (uint32_t)h;
}

// Sorted tiles: their canonical rank per table slot, and their coordinates.
__global__ void __launch_bounds__(256) k_tile_rank_scatter(const Key128* keys, const uint32_t* vals, i64 nt, i64 H,
                                                           int32_t* rank_of_slot, int4* utile, int32_t* flags) {
  const i64 s = (i64)blockIdx.x * 256 + threadIdx.x;
  if (s >= nt) return;
  const Key128 k = keys[s];
  if ((i64)vals[s] >= H) {  // consistency guard
    atomicOr(flags, kFlagInternal);
    return;
  }
  rank_of_slot[vals[s]] = (int32_t)s;
  const int32_t g = (int32_t)((k.hi << 4) | (k.lo >> 60));
  utile[s] = make_int4((int32_t)((k.lo >> 40) & 0xfffff) - kTileBias, (int32_t)((k.lo >> 20) & 0xfffff) - kTileBias,
                       (int32_t)(k.lo & 0xfffff) - kTileBias, g);
}

// Tile rank of a slot (-1 when out of range or unranked).
__device__ __forceinline__ int32_t slot_rank(const int32_t* rank_of_slot, i64 H, int32_t nt, i64 slot) {
  const int32_t t = (slot >= 0 && slot < H) ? rank_of_slot[slot] : -1;
  return (t >= 0 && t < nt) ? t : -1;
}

// Items per lane of one step of the record consumers.
constexpr int kPerLane = 4;  // kernels that merge through the block's LDS table (it holds twice a step's items)
constexpr int kPerBlock = 256 * kPerLane;
constexpr int kPerLaneWide = 8;
constexpr int kPerBlockWide = 256 * kPerLaneWide;
constexpr int kRecSplit = 2;  // consumer workgroups per region

// Every lower key sets its bit in its tile's candidate-lower mask (merged per
// mask word in LDS first: lower keys of nearby chunks repeat the same few
// lowers).
__global__ void __launch_bounds__(256) k_low_mark(const i64* low_cap, i64 last, const int32_t* region_lcnt, i64 cpw,
                                                  const int32_t* rank_of_slot, i64 H, int32_t nt, u64* tile_child,
                                                  int32_t* flags) {
  constexpr int V = kPerLane;
  __shared__ unsigned long long s_key[kBlockTable], s_val[kBlockTable];
  table_clear(s_key, s_val);
  const RegionPart p = region_part(region_lcnt, cpw, 1, kPerBlock);
  bool bad = false;
  for (int32_t j0 = p.first;; j0 += p.step) {
    i64 ld[V];
#pragma unroll
    for (int v = 0; v < V; ++v) ld[v] = low_cap[clamp_slot(p.base + j0 + step_item<V>(v), last)];
    if (j0 >= p.cnt) break;  // uniform
    bool ok[V];
    u64* word[V];
    u64 bits[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int32_t j = j0 + step_item<V>(v);
      const bool in = j < p.cnt;
      const i64 lk = in ? ld[v] : 0;
      const int32_t t = in ? slot_rank(rank_of_slot, H, nt, lk >> 15) : -1;
      ok[v] = in && t >= 0;
      bad |= in && t < 0;
      const int bit = (int)(lk & 32767);
      word[v] = ok[v] ? &tile_child[(i64)t * 512 + (bit >> 6)] : tile_child;
      bits[v] = 1ull << (bit & 63);
    }
    __syncthreads();  // the cleared table
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (ok[v]) table_or(s_key, s_val, word[v], bits[v]);
    __syncthreads();
    table_flush_clear(s_key, s_val);
  }
  if (bad) atomicOr(flags, kFlagInternal);
}

// Candidate lower of every record (tile base + rank of its bit in the tile's
// mask), the candidate's origin, and the record's leaf bit in the candidate's
// mask (merged per word in LDS). The candidate count is read on the device.
__global__ void __launch_bounds__(256) k_rec_cand(const int4* rec_cap, i64 last, const int32_t* region_cnt, i64 cpw,
                                                  const int32_t* rank_of_slot, i64 H, int32_t nt,
                                                  const u64* tile_child, const uint16_t* tile_prefix,
                                                  const int32_t* tile_lower_base, const int32_t* d_nc, int32_t* vcand,
                                                  int4* cand_origin, u64* cand_child, int32_t* flags) {
  constexpr int V = kPerLane;
  __shared__ unsigned long long s_key[kBlockTable], s_val[kBlockTable];
  table_clear(s_key, s_val);
  const int lane = threadIdx.x & (kWave - 1);
  const int32_t nc = *d_nc;
  const RegionPart p = region_part(region_cnt, cpw, kRecSplit, kPerBlock);
  bool bad = false;
  for (int32_t j0 = p.first;; j0 += p.step) {
    int4 ld[V];
#pragma unroll
    for (int v = 0; v < V; ++v) ld[v] = rec_cap[clamp_slot(p.base + j0 + step_item<V>(v), last)];
    if (j0 >= p.cnt) break;  // uniform
    bool ok[V];
    int4 r[V];
    int32_t t[V], c[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      ok[v] = j0 + step_item<V>(v) < p.cnt;
      r[v] = ok[v] ? ld[v] : make_int4(0, 0, 0, 0);
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
      t[v] = ok[v] ? slot_rank(rank_of_slot, H, nt, r[v].w) : 0;
      if (t[v] < 0) {
        bad = true;
        ok[v] = false;
        t[v] = 0;
      }
    }
    int w[V], bb[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int bit = (((r[v].x >> 7) & 31) * 32 + ((r[v].y >> 7) & 31)) * 32 + ((r[v].z >> 7) & 31);
      w[v] = bit >> 6;
      bb[v] = bit & 63;
    }
    int32_t base[V];
    uint16_t pre[V];
    u64 cw[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const i64 tt = t[v];
      base[v] = ok[v] ? tile_lower_base[tt] : 0;
      pre[v] = ok[v] ? tile_prefix[tt * 512 + w[v]] : 0;
      cw[v] = ok[v] ? tile_child[tt * 512 + w[v]] : 0ull;
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int32_t j = j0 + step_item<V>(v);
      c[v] = -1;
      if (ok[v]) {
        c[v] = base[v] + pre[v] + popc64(cw[v] & ((1ull << bb[v]) - 1));
        if (c[v] < 0 || c[v] >= nc || !((cw[v] >> bb[v]) & 1ull)) {
          bad = true;
          c[v] = -1;
          ok[v] = false;
        }
      }
      if (j < p.cnt) vcand[p.base + j] = c[v];
    }
    // one lane per run of equal candidates writes the candidate's origin
    u64* word[V];
    u64 bits[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int32_t cprev = __shfl_up(c[v], 1, kWave);
      if (ok[v] && (lane == 0 || cprev != c[v]))
        cand_origin[c[v]] = make_int4((r[v].x >> 7) * 128, (r[v].y >> 7) * 128, (r[v].z >> 7) * 128, t[v]);
      const int lb = (((r[v].x >> 3) & 15) * 16 + ((r[v].y >> 3) & 15)) * 16 + ((r[v].z >> 3) & 15);
      word[v] = ok[v] ? &cand_child[(i64)c[v] * 64 + (lb >> 6)] : cand_child;
      bits[v] = ok[v] ? 1ull << (lb & 63) : 0ull;
    }
    __syncthreads();  // the cleared table
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (ok[v]) table_or(s_key, s_val, word[v], bits[v]);
    __syncthreads();
    table_flush_clear(s_key, s_val);
  }
  if (bad) atomicOr(flags, kFlagInternal);
}

// Leaf words of the records (leaf = the candidate's first leaf + rank of the
// record's leaf bit in the candidate's mask), addressed slice-major: word x mod
// 8 of leaf l sits at (x mod 8) * L + l, so the records of a chunk (one x, and
// leaves that are neighbours in the canonical order) write a narrow range. A
// word can hold records of several chunks; one of them, the last to store its
// slot in owner[], writes the word with a plain store and the others OR into it
// afterwards (k_rec_word, k_rec_put<true>, k_rec_put<false> in that order); the
// leaf statistics pass then transposes the slices into the leaf masks.
__global__ void __launch_bounds__(256) k_rec_word(const int4* rec_cap, const int32_t* vcand, i64 last,
                                                  const int32_t* region_cnt, i64 cpw, const u64* cand_child,
                                                  const uint16_t* cand_prefix, const i64* cand_scan, i64 n_leaf,
                                                  i64* rec_word, int32_t* owner, int32_t* flags) {
  constexpr int V = kPerLaneWide;
  const RegionPart p = region_part(region_cnt, cpw, kRecSplit, kPerBlockWide);
  bool bad = false;
  for (int32_t j0 = p.first;; j0 += p.step) {
    int32_t lc[V];
    int4 lr[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const i64 q = clamp_slot(p.base + j0 + step_item<V>(v), last);
      lc[v] = vcand[q];
      lr[v] = rec_cap[q];
    }
    if (j0 >= p.cnt) break;  // uniform
    int4 r[V];
    int32_t c[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const bool in = j0 + step_item<V>(v) < p.cnt;
      c[v] = in ? lc[v] : -1;
      r[v] = in ? lr[v] : make_int4(0, 0, 0, 0);
    }
    int b[V];
    i64 sc[V];
    uint16_t pre[V];
    u64 cw[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int lb = (((r[v].x >> 3) & 15) * 16 + ((r[v].y >> 3) & 15)) * 16 + ((r[v].z >> 3) & 15);
      b[v] = lb & 63;
      const i64 cc = c[v];
      sc[v] = cc >= 0 ? cand_scan[cc] : 0;
      pre[v] = cc >= 0 ? cand_prefix[cc * 64 + (lb >> 6)] : 0;
      cw[v] = cc >= 0 ? cand_child[cc * 64 + (lb >> 6)] : 0ull;
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int32_t j = j0 + step_item<V>(v);
      if (j >= p.cnt) continue;
      i64 word = -1;
      if (c[v] >= 0) {
        const i64 leaf = (i64)(sc[v] & 0xffffffffll) + pre[v] + popc64(cw[v] & ((1ull << b[v]) - 1));
        if (leaf >= 0 && leaf < n_leaf && ((cw[v] >> b[v]) & 1ull)) word = (i64)(r[v].x & 7) * n_leaf + leaf;
      }
      rec_word[p.base + j] = word;
      if (word >= 0) owner[word] = (int32_t)(p.base + j);
      else bad = true;  // every record has its candidate lower and leaf
    }
  }
  if (bad) atomicOr(flags, kFlagInternal);
}

template <bool kOwner>
__global__ void __launch_bounds__(256) k_rec_put(const i64* rec_word, const u64* bits_cap, const int32_t* owner,
                                                 i64 last, const int32_t* region_cnt, i64 cpw, u64* slices) {
  constexpr int V = kPerLaneWide;
  const RegionPart p = region_part(region_cnt, cpw, kRecSplit, kPerBlockWide);
  for (int32_t j0 = p.first;; j0 += p.step) {
    i64 ld[V];
#pragma unroll
    for (int v = 0; v < V; ++v) ld[v] = rec_word[clamp_slot(p.base + j0 + step_item<V>(v), last)];
    if (j0 >= p.cnt) break;  // uniform
    i64 wd[V];
#pragma unroll
    for (int v = 0; v < V; ++v) wd[v] = j0 + step_item<V>(v) < p.cnt ? ld[v] : -1;
    int32_t o[V];
#pragma unroll
    for (int v = 0; v < V; ++v) o[v] = wd[v] >= 0 ? owner[wd[v]] : -1;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const i64 slot = p.base + j0 + step_item<V>(v);
      if (wd[v] < 0 || (o[v] == (int32_t)slot) != kOwner) continue;
      const u64 bits = bits_cap[slot];
      if (kOwner) slices[wd[v]] = bits;
      else atomicOr((unsigned long long*)&slices[wd[v]], (unsigned long long)bits);
    }
  }
}

// `n` consecutive device words read back with one synchronisation. The pinned
// staging buffer may still be the source of an earlier upload on the stream:
// the copy into it is ordered after that upload by the stream itself.
static void read_i32s(const int32_t* d, int n, hipStream_t s, int32_t* out) {
  int32_t* h = static_cast<int32_t*>(pinned_staging(64));
  hip_check(hipMemcpyAsync(h, d, 4 * (size_t)n, hipMemcpyDeviceToHost, s), "readback");
  hip_check(hipStreamSynchronize(s), "hipStreamSynchronize");
  for (int k = 0; k < n; ++k) out[k] = h[k];
}

static i64 pow2_at_least(i64 v) {
  i64 h = 1024;
  while (h < v) h <<= 1;
  return h;
}

tc_grid_batch* build_from_ijk(const int32_t* d_ijk, const int64_t* h_off, int32_t B, const OutAlloc& oa) {
  hipStream_t s = oa.stream;
  const i64 N = h_off[B];
  const i64 C = ceil_div(N, kRecChunk);
  const i64 G_max = std::max<i64>(1, (i64)device_cu_count() * kRecBlocksPerCu);
  const i64 cpw = std::max<i64>(1, ceil_div(C, G_max));  // chunks per region
  const i64 G = ceil_div(C, cpw);                          // regions (workgroups of the record pass)
  // A table of H_full >= 2N slots takes every possible tile at half load; the
  // first pass tries a small one, enough for all but scattered inputs.
  const i64 H_full = pow2_at_least(2 * N);

  // stage 1: records (by region), their tile slots, lower keys
  Arena a1(s);
  const size_t o_off = a1.reserve(8 * ((i64)B + 1));
  const size_t o_cg = a1.reserve(4 * (C + 1));
  const size_t o_cts = a1.reserve(4 * C);
  const size_t o_rec = a1.reserve(16 * N);
  const size_t o_bits = a1.reserve(8 * N);
  const size_t o_low = a1.reserve(8 * N);
  const size_t o_vc = a1.reserve(4 * N);
  const size_t o_rw = a1.reserve(8 * N);
  const size_t o_rc = a1.reserve(4 * G);
  const size_t o_rlc = a1.reserve(4 * G);
  const size_t o_ctl = a1.reserve(4 * kCtlWords);
  a1.commit();
  i64* d_off = a1.at<i64>(o_off);
  int32_t* chunk_g = a1.at<int32_t>(o_cg);
  int32_t* chunk_tslot = a1.at<int32_t>(o_cts);
  int4* rec_cap = a1.at<int4>(o_rec);
  u64* bits_cap = a1.at<u64>(o_bits);
  i64* low_cap = a1.at<i64>(o_low);
  int32_t* vcand = a1.at<int32_t>(o_vc);
  i64* rec_word = a1.at<i64>(o_rw);
  int32_t* region_cnt = a1.at<int32_t>(o_rc);
  int32_t* region_lcnt = a1.at<int32_t>(o_rlc);
  int32_t* ctl = a1.at<int32_t>(o_ctl);

  const size_t off_bytes = 8 * ((size_t)B + 1);
  void* h_stage = pinned_staging(off_bytes + 64);
  std::memcpy(h_stage, h_off, off_bytes);
  hip_check(hipMemcpyAsync(d_off, h_stage, off_bytes, hipMemcpyHostToDevice, s), "offsets upload");

  i64 H = std::min(H_full, kTileTableFirst);
  std::unique_ptr<Arena> a_tab;
  int32_t* table = nullptr;
  int32_t h_ctl[kCtlWords] = {};
  for (;;) {
    a_tab.reset();  // a smaller table of a first try goes back to the cache
    a_tab.reset(new Arena(s));
    const size_t o_tab = a_tab->reserve(4 * H);
    a_tab->commit();
    table = a_tab->at<int32_t>(o_tab);
    fill_i32(ctl, 0, kCtlWords, nullptr, 1, s);
    fill_i32(table, -1, H, nullptr, 1, s);
    launch("k_chunk_prep", k_chunk_prep, ceil_div(C + 1, 256), 256, s, d_ijk, (const i64*)d_off, B, N, C, chunk_g,
           chunk_tslot, table, H, ctl);
    launch("k_ijk_records", k_ijk_records, G, 256, s, d_ijk, (const i64*)d_off, B, N, (const int32_t*)chunk_g,
           (const int32_t*)chunk_tslot, C, cpw, rec_cap, bits_cap, low_cap, region_cnt, region_lcnt, table, H, ctl);
    read_i32s(ctl, kCtlWords, s, h_ctl);
    if ((h_ctl[2] & kRetryFlag) && H < H_full) {
      // every tile holds a record: 2R slots take them all at half load
      H = std::min(H_full, std::max(2 * H, pow2_at_least(2 * (i64)h_ctl[5])));
      continue;
    }
    break;
  }
  if (h_ctl[2] != 0) throw Error(TC_ERR_INTERNAL, "from_ijk: record pass consistency check failed");
  const i64 R = h_ctl[5];
  const int32_t nt = h_ctl[1];
  const i64 NL = h_ctl[4];
  if (R < 0 || R > N || nt < 0 || nt > R || NL < 0 || NL > R)
    throw Error(TC_ERR_INTERNAL, "from_ijk: record counts out of range");

  // stage 2: sorted unique tiles, candidate lowers (at most one per lower key),
  // their leaves and the node counts
  Arena a2(s);
  const size_t o_keys = a2.reserve(sizeof(Key128) * nt);
  const size_t o_vals = a2.reserve(4 * (i64)nt);
  const size_t o_rank = a2.reserve(4 * H);
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
  const size_t o_corig = a2.reserve(16 * NL);
  const size_t o_cchild = a2.reserve(512 * NL);
  const size_t o_cpre = a2.reserve(128 * NL);
  const size_t o_clc = a2.reserve(8 * NL);
  const size_t o_lb = a2.reserve(8 * (NL + 1));
  const size_t o_ginfo = a2.reserve(4 * 6 * (i64)B);
  const size_t o_rb = a2.reserve(4 * (4 + 3 * (i64)B));
  const size_t o_stmp = a2.reserve(std::max(scan_tmp_bytes(nt, 4), scan_tmp_bytes(NL, 8)));
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
  ts.cap_cands = NL;
  ts.cand_origin = a2.at<int4>(o_corig);
  ts.cand_child = a2.at<u64>(o_cchild);
  ts.cand_prefix = a2.at<uint16_t>(o_cpre);
  ts.cand_counts = a2.at<i64>(o_clc);
  ts.cand_scan = a2.at<i64>(o_lb);
  ts.grid_info = a2.at<int32_t>(o_ginfo);
  ts.readback = a2.at<int32_t>(o_rb);
  ts.scan_tmp = a2.at<char>(o_stmp);
  ts.flags = ts.readback;
  Key128* keys = a2.at<Key128>(o_keys);
  uint32_t* vals = a2.at<uint32_t>(o_vals);
  int32_t* rank_of_slot = a2.at<int32_t>(o_rank);

  fill_i32(ts.readback, 0, 1, nullptr, 1, s);
  fill_i32(ts.d_num_tiles, nt, 1, nullptr, 1, s);
  launch("k_tile_collect", k_tile_collect, ceil_div(H, 256), 256, s, (const int32_t*)table, H, d_ijk,
         (const i64*)d_off, B, nt, ctl + 3, keys, vals, ts.flags);
  sort_pairs_128(keys, vals, nt, tile_key_bits(B), s);
  launch("k_tile_rank_scatter", k_tile_rank_scatter, ceil_div(nt, 256), 256, s, (const Key128*)keys,
         (const uint32_t*)vals, (i64)nt, H, rank_of_slot, ts.utile, ts.flags);
  tree_tile_ranges(ts, B, s);
  fill_u64(ts.tile_child, 0, 512 * (i64)nt, nullptr, 1, s);
  launch("k_low_mark", k_low_mark, G, 256, s, (const i64*)low_cap, N - 1, (const int32_t*)region_lcnt, cpw,
         (const int32_t*)rank_of_slot, H, nt, ts.tile_child, ts.flags);
  tree_rank_tiles(ts, s);
  fill_u64(ts.cand_child, 0, 64 * NL, ts.d_num_cands, 64, s);
  launch("k_rec_cand", k_rec_cand, G * kRecSplit, 256, s, (const int4*)rec_cap, N - 1, (const int32_t*)region_cnt, cpw,
         (const int32_t*)rank_of_slot, H, nt, (const u64*)ts.tile_child, (const uint16_t*)ts.tile_prefix,
         (const int32_t*)ts.tile_lower_base, (const int32_t*)ts.d_num_cands, vcand, ts.cand_origin, ts.cand_child,
         ts.flags);
  a_tab.reset();
  const size_t rb_bytes = 4 * (4 + 3 * (size_t)B);
  int32_t* h_rb = static_cast<int32_t*>(pinned_staging(rb_bytes));
  if (!tree_counts(ts, B, s, h_rb))  // else the counts stage wrote the words into h_rb
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
    const size_t o_own = post.reserve(4 * 8 * L);
    const size_t o_sl = post.reserve(8 * 8 * L);
    post.commit();
    int32_t* owner = post.at<int32_t>(o_own);
    u64* slices = post.at<u64>(o_sl);
    tree_write_nodes(ts, ov, post.at<int32_t>(o_lc), s);
    fill_u64(slices, 0, 8 * L, nullptr, 1, s);
    launch("k_rec_word", k_rec_word, G * kRecSplit, 256, s, (const int4*)rec_cap, (const int32_t*)vcand, N - 1,
           (const int32_t*)region_cnt, cpw, (const u64*)ts.cand_child, (const uint16_t*)ts.cand_prefix,
           (const i64*)ts.cand_scan, L, rec_word, owner, ts.flags);
    launch("k_rec_put<owner>", k_rec_put<true>, G * kRecSplit, 256, s, (const i64*)rec_word, (const u64*)bits_cap,
           (const int32_t*)owner, N - 1, (const int32_t*)region_cnt, cpw, slices);
    launch("k_rec_put<merge>", k_rec_put<false>, G * kRecSplit, 256, s, (const i64*)rec_word, (const u64*)bits_cap,
           (const int32_t*)owner, N - 1, (const int32_t*)region_cnt, cpw, slices);
    tree_leaf_stats(ov, slices, post.at<uint32_t>(o_box), post.at<int32_t>(o_inrun), post.at<i64>(o_part), s);
    apply_debug_inject(ts.flags, s);  // k_rec_word's checks ran after the readback: finalize copies the word
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
