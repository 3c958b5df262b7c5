// One batched topology pass over every source leaf of every member
// (PR page "Batched leaf-mask topology construction for generated conv grids",
// section 1: emission over all source leaves of all members, canonical order,
// dedup, one readback, one allocation, batched writers; section 2: box-dilate
// [-1,1]^3 and the pads {-1,0}^3 / {0,1}^3 via per-axis bit shifts).
//
// Mask layout: leaf bit n = x*64 + y*8 + z, i.e. word x, byte y, bit z; lower
// child bit (x*16+y)*16+z; upper child bit (x*32+y)*32+z.
//
// Stages (sizes are host-known bounds, so nothing waits before the readback):
//   tiles   each source upper proposes its target root tiles; one small sort of
//           the (grid, tile) keys and a head-flag scan give the unique tiles;
//   lowers  each source lower sets its candidate target lowers in the target
//           tile's 32^3 mask; ranks in those masks number the candidates;
//   leaves  every non-empty target leaf gets its bit in its target lower's 16^3
//           mask: refine from the source side (two workgroups per source
//           lower, one per x half, mark their leaves' children in LDS copies
//           of the target lowers' masks); coarsen from the target side (one
//           wave per candidate lower ORs 2x2x2 blocks of its source lowers'
//           masks); the box ops from the target side too (workgroups loop
//           over candidate lowers, collect the facing source leaves of each
//           one's <= 27 source lowers and OR their reach into an LDS mask); no
//           device atomics on masks in any case;
//   counts  popcounts and scans give per-grid counts -> the single readback;
//   writers node records, then every output leaf gathers its mask from the
//           (at most 1 / 8 / 27) source leaves that feed it (no atomics); a
//           consistency check that fails there sets a flag word that is read
//           back with the batch's voxel total.
#include <atomic>

#include "device.hpp"
#include "internal.hpp"

namespace tc {

constexpr u64 kZ0 = 0x0101010101010101ull;  // z = 0 bit of every (x, y) row
constexpr u64 kZ7 = 0x8080808080808080ull;  // z = 7 bit of every row

// The pass's flag word starts from the source batch's status word.
__global__ void k_flags_from_source(int32_t* flags, const int32_t* src_status) {
  if (threadIdx.x == 0) flags[0] = src_status[0] != 0 ? kFlagSource : 0;
}

struct I3 {
  i64 x, y, z;
};

__device__ __forceinline__ I3 octant(int j) { return {(j >> 2) & 1, (j >> 1) & 1, j & 1}; }
__device__ __forceinline__ int octant_index(i64 x, i64 y, i64 z) { return (int)((x << 2) | (y << 1) | z); }

// j -> box offset of the op (DILATE: base-3 digits minus one; pads: sign * bits).
__device__ __forceinline__ I3 box_offset(int j, int op) {
  if (op == TC_OP_DILATE) return {j / 9 - 1, (j / 3) % 3 - 1, j % 3 - 1};
  const i64 s = op == TC_OP_PAD_NEG ? -1 : 1;
  return {s * ((j >> 2) & 1), s * ((j >> 1) & 1), s * (j & 1)};
}
__device__ __forceinline__ int box_index(i64 x, i64 y, i64 z, int op) {
  if (op == TC_OP_DILATE) return (int)((x + 1) * 9 + (y + 1) * 3 + (z + 1));
  const i64 s = op == TC_OP_PAD_NEG ? -1 : 1;
  return (int)(((s * x) << 2) | ((s * y) << 1) | (s * z));
}
__device__ __forceinline__ int index27(i64 x, i64 y, i64 z) { return (int)((x + 1) * 9 + (y + 1) * 3 + (z + 1)); }

__device__ __forceinline__ bool tile_ok(i64 t) { return t >= -kTileBias && t < kTileBias; }
__device__ __forceinline__ bool lower_ok(i64 k) { return k >= -(1ll << 24) && k < (1ll << 24); }
__device__ __forceinline__ bool leaf_ok(i64 l) { return l >= -(1ll << 28) && l < (1ll << 28); }

__device__ __forceinline__ void set_flag(int32_t* flags, int f) { atomicOr(flags, f); }

// One wave holds the 64 words of candidate c's 16^3 leaf mask (lane = word):
// writes the word, the word's exclusive popcount prefix and the candidate's
// packed count (leaves | non-empty << 32). Every lane of the wave must call it.
__device__ __forceinline__ void store_candidate(i64 c, u64 word, u64* cand_child, uint16_t* cand_prefix,
                                                i64* cand_counts) {
  const int lane = threadIdx.x & (kWave - 1);
  const int cnt = popc64(word);
  const int inc = wave_incl_scan(cnt);
  cand_child[c * 64 + lane] = word;
  cand_prefix[c * 64 + lane] = (uint16_t)(inc - cnt);
  if (lane == kWave - 1) cand_counts[c] = (i64)inc | ((i64)(inc > 0 ? 1 : 0) << 32);
}

// ------------------------------------------------------------------ stage: tiles
__global__ void __launch_bounds__(256) k_tile_candidates(const int4* upper_origin, i64 n, int op, int m,
                                                         Key128* keys, uint32_t* vals) {
  const i64 i = (i64)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const i64 u = i / m;
  const int j = (int)(i % m);
  const int4 o = upper_origin[u];
  const i64 tx = o.x >> 12, ty = o.y >> 12, tz = o.z >> 12;
  I3 t;
  if (op == TC_OP_REFINE) {
    const I3 q = octant(j);
    t = {2 * tx + q.x, 2 * ty + q.y, 2 * tz + q.z};
  } else if (op == TC_OP_COARSEN) {
    t = {tx >> 1, ty >> 1, tz >> 1};
  } else {
    const I3 e = box_offset(j, op);
    t = {tx + e.x, ty + e.y, tz + e.z};
  }
  Key128 k{~0ull, ~0ull};
  if (tile_ok(t.x) && tile_ok(t.y) && tile_ok(t.z)) {
    const u64 g = (uint32_t)o.w;
    k.lo = ((g & 15ull) << 60) | ((u64)(t.x + kTileBias) << 40) | ((u64)(t.y + kTileBias) << 20) |
           (u64)(t.z + kTileBias);
    k.hi = g >> 4;
  }
  keys[i] = k;
  vals[i] = (uint32_t)i;
}

__device__ __forceinline__ bool key_valid(const Key128& k) { return !(k.lo == ~0ull && k.hi == ~0ull); }

__global__ void __launch_bounds__(256) k_tile_heads(const Key128* keys, i64 n, int32_t* head) {
  const i64 i = (i64)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const Key128 k = keys[i];
  bool h = key_valid(k);
  if (h && i > 0) {
    const Key128 p = keys[i - 1];
    h = !(p.lo == k.lo && p.hi == k.hi);
  }
  head[i] = h ? 1 : 0;
}

__global__ void __launch_bounds__(256) k_tile_scatter(const Key128* keys, const uint32_t* vals, const int32_t* head,
                                                      const int32_t* excl, i64 n, int4* utile, int32_t* tile_of_cand,
                                                      int32_t* flags) {
  const i64 i = (i64)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const Key128 k = keys[i];
  const uint32_t v = vals[i];
  if ((i64)v >= n) {
    set_flag(flags, kFlagInternal);
    return;
  }
  if (!key_valid(k)) {
    tile_of_cand[v] = -1;
    return;
  }
  const int32_t t = excl[i] + head[i] - 1;
  if (t < 0 || t >= n) {
    set_flag(flags, kFlagInternal);
    return;
  }
  tile_of_cand[v] = t;
  if (head[i]) {
    const int32_t g = (int32_t)((k.hi << 4) | (k.lo >> 60));
    const int32_t x = (int32_t)((k.lo >> 40) & 0xfffff) - kTileBias;
    const int32_t y = (int32_t)((k.lo >> 20) & 0xfffff) - kTileBias;
    const int32_t z = (int32_t)(k.lo & 0xfffff) - kTileBias;
    utile[t] = make_int4(x, y, z, g);
  }
}

// ------------------------------------------------------------------ candidate pruning
// A source node proposes target j (a neighbour for box ops, a child octant for
// refine) only when one of its own children can reach it: for box offset e,
// a child on the boundary face/edge/corner that e points to; for refine, a child
// inside octant j. Coarsen always proposes its single target. The leaf-level
// marking only ever reaches targets that pass this test, because the child it
// comes from is itself the witness.

// Lower node: 16^3 leaves in 64 words; word x*4 + (y >> 2), bit (y & 3)*16 + z.
__device__ __forceinline__ bool lower_reaches(const u64* m, int op, int j) {
  if (op == TC_OP_COARSEN) return true;
  if (op == TC_OP_REFINE) {
    const I3 q = octant(j);
    const u64 zm = q.z ? 0xff00ff00ff00ff00ull : 0x00ff00ff00ff00ffull;
    u64 acc = 0;
    for (i64 x = 8 * q.x; x < 8 * q.x + 8; ++x) acc |= m[x * 4 + 2 * q.y] | m[x * 4 + 2 * q.y + 1];
    return (acc & zm) != 0;
  }
  const I3 e = box_offset(j, op);
  if (e.x == 0 && e.y == 0 && e.z == 0) return true;
  const int x0 = e.x > 0 ? 15 : 0, x1 = e.x < 0 ? 0 : 15;
  const u64 zm = e.z > 0 ? 0x8000800080008000ull : (e.z < 0 ? 0x0001000100010001ull : ~0ull);
  u64 acc = 0;
  for (int x = x0; x <= x1; ++x) {
    if (e.y > 0) acc |= m[x * 4 + 3] & 0xffff000000000000ull;  // y = 15
    else if (e.y < 0) acc |= m[x * 4] & 0xffffull;              // y = 0
    else acc |= m[x * 4] | m[x * 4 + 1] | m[x * 4 + 2] | m[x * 4 + 3];
  }
  return (acc & zm) != 0;
}

// Reach set contributed by word w of a lower's 16^3 leaf mask, in the same
// encoding as upper_word_reach (27-bit box offsets, or 8-bit child octants for
// refine); the union over the 64 words equals lower_reaches for every target.
__device__ __forceinline__ uint32_t product27(uint32_t ax, uint32_t ay, uint32_t az);
__device__ __forceinline__ uint32_t axis_set(bool lo_face, bool hi_face);
__device__ __forceinline__ uint32_t lower_word_reach(u64 word, int w, int op) {
  if (!word) return 0;
  const int x = w >> 2, yq = w & 3;
  if (op == TC_OP_REFINE) {
    const int qx = x >> 3, qy = yq >> 1;
    uint32_t code = 0;
    if (word & 0x00ff00ff00ff00ffull) code |= 1u << octant_index(qx, qy, 0);
    if (word & 0xff00ff00ff00ff00ull) code |= 1u << octant_index(qx, qy, 1);
    return code;
  }
  const uint32_t ax = axis_set(x == 0, x == 15);
  uint32_t code = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t v = (uint32_t)(word >> (16 * r)) & 0xffffu;
    if (!v) continue;
    const int y = yq * 4 + r;
    code |= product27(ax, axis_set(y == 0, y == 15), axis_set((v & 1u) != 0, (v >> 15) != 0));
  }
  return code;
}

// 27-bit box-offset set -> the op's candidate numbering (identity for dilate).
__device__ __forceinline__ uint32_t box_code_for_op(uint32_t code27, int op, int m) {
  if (op == TC_OP_DILATE) return code27;
  uint32_t c = 0;
  for (int j = 0; j < m; ++j) {
    const I3 e = box_offset(j, op);
    c |= ((code27 >> index27(e.x, e.y, e.z)) & 1u) << j;
  }
  return c;
}

// Upper node: 32^3 lowers in 512 words; word x*16 + (y >> 1), bit (y & 1)*32 + z.
// Reach set of the lowers present in word w. Box ops: a 27-bit set indexed like
// index27 (each lower reaches the product of its per-axis offset sets, {0} plus
// -1 / +1 on the low / high face); refine: the 8-bit set of child octants.
__device__ __forceinline__ uint32_t axis_set(bool lo_face, bool hi_face) {
  return 2u | (lo_face ? 1u : 0u) | (hi_face ? 4u : 0u);  // bit e + 1
}
__device__ __forceinline__ uint32_t product27(uint32_t ax, uint32_t ay, uint32_t az) {
  uint32_t yz = 0, xyz = 0;
#pragma unroll
  for (int b = 0; b < 3; ++b)
    if ((ay >> b) & 1u) yz |= az << (3 * b);
#pragma unroll
  for (int b = 0; b < 3; ++b)
    if ((ax >> b) & 1u) xyz |= yz << (9 * b);
  return xyz;
}
__device__ __forceinline__ uint32_t upper_word_reach(u64 word, int w, int op) {
  if (!word) return 0;
  const int ux = w >> 4;
  if (op == TC_OP_REFINE) {
    const int qx = ux >> 4, qy = (w & 15) >> 3;
    uint32_t code = 0;
    if (word & 0x0000ffff0000ffffull) code |= 1u << octant_index(qx, qy, 0);
    if (word & 0xffff0000ffff0000ull) code |= 1u << octant_index(qx, qy, 1);
    return code;
  }
  const uint32_t ax = axis_set(ux == 0, ux == 31);
  uint32_t code = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t v = (uint32_t)(word >> (32 * h));
    if (!v) continue;
    const int uy = 2 * (w & 15) + h;
    code |= product27(ax, axis_set(uy == 0, uy == 31), axis_set((v & 1u) != 0, (v >> 31) != 0));
  }
  return code;
}

// Reach set of every source node, one wave per node (uppers: 8 mask words per
// lane; lowers: one), for batches too large to do it inside the single-workgroup
// stages. Workgroups from `lo_block` on take the lowers of a second node set
// (mask_lo, n_lo, reach_lo), so that the uppers' and the lowers' sets come from
// one launch.
__global__ void __launch_bounds__(256) k_node_reach(const u64* mask, i64 n_nodes, int words, int op, int m,
                                                    uint32_t* reach, i64 lo_block, const u64* mask_lo, i64 n_lo,
                                                    uint32_t* reach_lo) {
  i64 u = (i64)blockIdx.x * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if ((i64)blockIdx.x >= lo_block) {  // uniform per block: the second set (lowers)
    u = ((i64)blockIdx.x - lo_block) * 4 + threadIdx.x / kWave;
    mask = mask_lo;
    n_nodes = n_lo;
    words = 64;
    reach = reach_lo;
  }
  if (u >= n_nodes) return;  // uniform per wave
  uint32_t code = 0;
  if (words == 512) {
#pragma unroll
    for (int k = 0; k < 8; ++k) code |= upper_word_reach(mask[u * 512 + k * kWave + lane], k * kWave + lane, op);
  } else {
    code = lower_word_reach(mask[u * 64 + lane], lane, op);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) code |= (uint32_t)__shfl_xor((int)code, d, kWave);
  if (lane == 0) reach[u] = op == TC_OP_REFINE ? code : box_code_for_op(code, op, m);
}

// Box ops, voxel-exact faces: reach sets of every source upper and lower from
// which faces of the node hold a voxel (the node's voxels at local coordinate 0
// or at the far end, per axis). A node reaches the neighbour at offset e only if
// every axis with e != 0 has a voxel on that face, so the product of the per-axis
// sets stays a superset of the true targets while dropping the neighbours that
// the child-bit sets above add whenever a child merely sits on a face. One
// workgroup per source upper; its threads take the upper's leaves (contiguous,
// two at a time in flight). A leaf's position in its lower and tile comes from
// its origin alone; the lowers' face bits gather in LDS (an upper has at most
// kBoxReachLowers lowers here). Face bits: 2a for the low face of axis a, 2a + 1
// for the high face.
constexpr int kBoxReachLowers = 512;

__device__ __forceinline__ uint32_t faces_to_code(uint32_t f, int op, int m) {
  const uint32_t code = product27(axis_set(f & 1u, f & 2u), axis_set(f & 4u, f & 8u), axis_set(f & 16u, f & 32u));
  return box_code_for_op(code, op, m);
}

// Faces of the node (side `side` = 8 << level voxels, origins aligned to it)
// that leaf origin o with mask words w touches.
__device__ __forceinline__ uint32_t leaf_faces(const int4 o, const u64 w[8], int side) {
  const u64 all = w[0] | w[1] | w[2] | w[3] | w[4] | w[5] | w[6] | w[7];
  const int m = side - 1, far = side - 8;
  const int px = o.x & m, py = o.y & m, pz = o.z & m;
  uint32_t f = 0;
  if (px == 0 && w[0]) f |= 1u;
  if (px == far && w[7]) f |= 2u;
  if (py == 0 && (all & 0xffull)) f |= 4u;
  if (py == far && (all & 0xff00000000000000ull)) f |= 8u;
  if (pz == 0 && (all & kZ0)) f |= 16u;
  if (pz == far && (all & kZ7)) f |= 32u;
  return f;
}

__global__ void __launch_bounds__(256) k_box_reach(const int32_t* upper_first, int32_t n_upper,
                                                   const int32_t* lower_first, int32_t n_lower,
                                                   const int4* leaf_origin, const int32_t* leaf_parent,
                                                   const u64* leaf_mask, int32_t n_leaf, int op, int m,
                                                   uint32_t* upper_reach, uint32_t* lower_reach) {
  __shared__ uint32_t s_lface[kBoxReachLowers];
  __shared__ uint32_t s_face;
  const int u = blockIdx.x;
  const int32_t l0 = upper_first[u], l1 = u + 1 < n_upper ? upper_first[u + 1] : n_lower;
  for (int k = threadIdx.x; k < l1 - l0; k += 256) s_lface[k] = 0;
  if (threadIdx.x == 0) s_face = 0;
  const int32_t f0 = lower_first[l0], f1 = l1 < n_lower ? lower_first[l1] : n_leaf;
  __syncthreads();
  for (int32_t f = f0 + threadIdx.x; f < f1; f += 2 * 256) {
    int4 o[2];
    int32_t lp[2];
    u64 w[2][8];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int32_t fq = min(f + q * 256, f1 - 1);
      o[q] = leaf_origin[fq];
      lp[q] = leaf_parent[fq];
#pragma unroll
      for (int k = 0; k < 8; ++k) w[q][k] = leaf_mask[(i64)fq * 8 + k];
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (f + q * 256 >= f1) continue;
      const uint32_t lf = leaf_faces(o[q], w[q], 128);
      const uint32_t tf = leaf_faces(o[q], w[q], 4096);
      const int32_t li = lp[q] - l0;
      if (lf && li >= 0 && li < l1 - l0) atomicOr(&s_lface[li], lf);
      if (tf) atomicOr(&s_face, tf);
    }
  }
  __syncthreads();
  for (int k = threadIdx.x; k < l1 - l0; k += 256) lower_reach[l0 + k] = faces_to_code(s_lface[k], op, m);
  if (threadIdx.x == 0) upper_reach[u] = faces_to_code(s_face, op, m);
}

// ------------------------------------------------------------------ stage: tiles, fused (small batches)
// At most 4096 tile candidates: one workgroup builds the reach set of every
// source upper, compacts the reachable in-range candidates, brings their
// (grid, tile) keys into canonical order without duplicates (a rank sort for
// at most 64 keys; above that an LDS bitmap over the batch's key space when it
// is small, else a rank sort up to 256 keys or an LDS bitonic network, then
// head flags and a scan), scatters the unique tiles and every candidate's tile index, writes the
// per-grid tile ranges and, when asked (few tiles), zeroes the unique tiles'
// lower bitmaps; more tiles get a wide fill.
constexpr int kTilesMax = 4096;
constexpr int kTilesThreads = 1024;
constexpr int kTilesItems = kTilesMax / kTilesThreads;
// keys sorted by rank counting (each of T = 1024 / K threads per key scans K / T
// keys: a serial chain of LDS reads); more keys go through a bitonic network,
// which is faster from a few hundred keys on (at 388 keys the rank sort took
// twice as long)
constexpr int kRankMax = 256;
constexpr int kSegMax = 128;  // keys per grid for the per-grid rank sort
constexpr i64 kTileBits = 65536;  // mixed-radix (grid, tile) key space handled by an LDS bitmap

// LDS of the tile stage, carved from one block so that the fused node stage
// can reuse it for the lower stage (offsets in bytes, 16-byte aligned).
constexpr int kTL_hi = 0;
constexpr int kTL_lo = kTL_hi + 8 * kTilesMax;
constexpr int kTL_v = kTL_lo + 8 * kTilesMax;
constexpr int kTL_g = kTL_v + 4 * kTilesMax;
constexpr int kTL_bits = kTL_g + 4 * kTilesMax;
constexpr int kTL_wpre = kTL_bits + 8 * (kTileBits / 64);
constexpr int kTL_cnt = kTL_wpre + 4 * (kTileBits / 64);
constexpr int kTL_wave = kTL_cnt + 4 * kTilesThreads;
constexpr int kTL_rng = kTL_wave + 4 * (kTilesThreads / kWave);
constexpr int kTL_nt = kTL_rng + 4 * 8;
constexpr int kTilesLds = kTL_nt + 16;

__device__ __forceinline__ void tiles_small_body(const int4* upper_origin, const u64* upper_mask, int32_t n_upper,
                                                 int op, int m, int32_t B, int4* utile, int32_t* tile_of_cand,
                                                 int32_t* d_num_tiles, int32_t* grid_tile_begin, u64* tile_child,
                                                 int zero_child, const uint32_t* upper_reach, int32_t* readback,
                                                 const int32_t* src_status, char* lds) {
  u64* s_hi = reinterpret_cast<u64*>(lds + kTL_hi);
  u64* s_lo = reinterpret_cast<u64*>(lds + kTL_lo);
  uint32_t* s_v = reinterpret_cast<uint32_t*>(lds + kTL_v);
  int32_t* s_g = reinterpret_cast<int32_t*>(lds + kTL_g);  // reach set per upper first, grid per unique tile later
  int32_t* s_wave = reinterpret_cast<int32_t*>(lds + kTL_wave);
  uint32_t* s_code = reinterpret_cast<uint32_t*>(s_g);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int n = n_upper * m;
  int32_t* s_rng = reinterpret_cast<int32_t*>(lds + kTL_rng);  // min x, y, z, max x, y, z of the kept candidates' tiles
  // the candidates' upper origins, issued first: no wait on the reach sets
  int4 org[kTilesItems];
#pragma unroll
  for (int k = 0; k < kTilesItems; ++k) org[k] = upper_origin[min(tid * kTilesItems + k, n - 1) / m];  // n >= 1
  if (tid == 0) {
    readback[0] = src_status[0] != 0 ? kFlagSource : 0;  // a flawed source fails the pass
    for (int a = 0; a < 3; ++a) {
      s_rng[a] = INT32_MAX;
      s_rng[3 + a] = INT32_MIN;
    }
  }
  if (op != TC_OP_COARSEN && upper_reach) {  // computed by k_node_reach
    for (int u = tid; u < n_upper; u += kTilesThreads) s_code[u] = upper_reach[u];
  } else if (op != TC_OP_COARSEN) {
    // each wave reduces kUppersPerWave uppers at a time, so that many mask loads
    // are in flight at once
    constexpr int kUppersPerWave = 4;
    constexpr int kWaves = kTilesThreads / kWave;
    for (int u0 = wv * kUppersPerWave; u0 < n_upper; u0 += kWaves * kUppersPerWave) {
      u64 words[kUppersPerWave][8];
#pragma unroll
      for (int v = 0; v < kUppersPerWave; ++v)
#pragma unroll
        for (int k = 0; k < 8; ++k)
          words[v][k] = upper_mask[(i64)min(u0 + v, n_upper - 1) * 512 + k * kWave + lane];  // clamped: no wait per load
#pragma unroll
      for (int v = 0; v < kUppersPerWave; ++v) {
        uint32_t code = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) code |= upper_word_reach(words[v][k], k * kWave + lane, op);
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) code |= (uint32_t)__shfl_xor((int)code, d, kWave);
        if (lane == 0 && u0 + v < n_upper) s_code[u0 + v] = op == TC_OP_REFINE ? code : box_code_for_op(code, op, m);
      }
    }
  }
  __syncthreads();
  // keys of the kept candidates (blocked: thread tid owns tid*4 .. tid*4+3);
  // the origins are loaded first, at clamped indices, all in flight at once
  u64 khi[kTilesItems], klo[kTilesItems];
  int keep[kTilesItems];
  int nkeep = 0;
#pragma unroll
  for (int k = 0; k < kTilesItems; ++k) {
    const int i = tid * kTilesItems + k;
    keep[k] = 0;
    khi[k] = klo[k] = 0;
    if (i < n) {
      const int u = i / m, j = i % m;
      const int4 o = org[k];
      const i64 tx = o.x >> 12, ty = o.y >> 12, tz = o.z >> 12;
      I3 t;
      bool reach = true;
      if (op == TC_OP_REFINE) {
        const I3 q = octant(j);
        t = {2 * tx + q.x, 2 * ty + q.y, 2 * tz + q.z};
        reach = (s_code[u] >> j) & 1u;
      } else if (op == TC_OP_COARSEN) {
        t = {tx >> 1, ty >> 1, tz >> 1};
      } else {
        const I3 e = box_offset(j, op);
        t = {tx + e.x, ty + e.y, tz + e.z};
        reach = (s_code[u] >> j) & 1u;
      }
      if (reach && tile_ok(t.x) && tile_ok(t.y) && tile_ok(t.z)) {
        const u64 g = (uint32_t)o.w;
        klo[k] = ((g & 15ull) << 60) | ((u64)(t.x + kTileBias) << 40) | ((u64)(t.y + kTileBias) << 20) |
                 (u64)(t.z + kTileBias);
        khi[k] = g >> 4;
        keep[k] = 1;
      } else {
        tile_of_cand[i] = -1;
      }
    }
    nkeep += keep[k];
  }
  int K;
  int pos = block_excl_scan<int, kTilesThreads>(nkeep, s_wave, K);
#pragma unroll
  for (int k = 0; k < kTilesItems; ++k) {
    if (keep[k]) {
      s_hi[pos] = khi[k];
      s_lo[pos] = klo[k];
      s_v[pos] = (uint32_t)(tid * kTilesItems + k);
      ++pos;
    }
  }
  int32_t& s_nt = *reinterpret_cast<int32_t*>(lds + kTL_nt);
  // More than 64 keys: the (grid, tile) keys of the kept candidates, relative to
  // the batch's tile ranges, index a mixed-radix space of S = B * Rx * Ry * Rz
  // points in canonical order. When S is at most kTileBits, one bit per
  // candidate in an LDS bitmap replaces the sort: the set bits are the unique
  // tiles in order, and a popcount prefix gives every candidate its tile (whose
  // record every candidate of it writes, with the same value).
  u64* s_bits = reinterpret_cast<u64*>(lds + kTL_bits);
  int32_t* s_wpre = reinterpret_cast<int32_t*>(lds + kTL_wpre);
  if (K > kWave) {  // uniform
    {
      int rmin[3] = {INT32_MAX, INT32_MAX, INT32_MAX}, rmax[3] = {INT32_MIN, INT32_MIN, INT32_MIN};
#pragma unroll
      for (int k = 0; k < kTilesItems; ++k) {
        if (!keep[k]) continue;
        const int tv[3] = {(int)((klo[k] >> 40) & 0xfffff) - kTileBias, (int)((klo[k] >> 20) & 0xfffff) - kTileBias,
                           (int)(klo[k] & 0xfffff) - kTileBias};
        for (int a = 0; a < 3; ++a) {
          rmin[a] = min(rmin[a], tv[a]);
          rmax[a] = max(rmax[a], tv[a]);
        }
      }
#pragma unroll
      for (int a = 0; a < 3; ++a) {
        rmin[a] = wave_min_i32(rmin[a]);
        rmax[a] = wave_max_i32(rmax[a]);
      }
      if (lane == 0 && rmin[0] <= rmax[0]) {
        for (int a = 0; a < 3; ++a) {
          atomicMin(&s_rng[a], rmin[a]);
          atomicMax(&s_rng[3 + a], rmax[a]);
        }
      }
    }
    __syncthreads();
    const i64 R64[3] = {(i64)s_rng[3] - s_rng[0] + 1, (i64)s_rng[4] - s_rng[1] + 1, (i64)s_rng[5] - s_rng[2] + 1};
    i64 S = B;
    for (int a = 0; a < 3 && S <= kTileBits; ++a) S *= R64[a];
    if (S <= kTileBits) {  // every index below fits in 32 bits
      const int R[3] = {(int)R64[0], (int)R64[1], (int)R64[2]};
      const int nw = (int)((S + 63) >> 6);
      for (int w = tid; w < nw; w += kTilesThreads) s_bits[w] = 0;
      __syncthreads();
      int pk[kTilesItems];
#pragma unroll
      for (int k = 0; k < kTilesItems; ++k) {
        pk[k] = -1;
        if (!keep[k]) continue;
        const int g = (int)((khi[k] << 4) | (klo[k] >> 60));
        const int x = (int)((klo[k] >> 40) & 0xfffff) - kTileBias - s_rng[0];
        const int y = (int)((klo[k] >> 20) & 0xfffff) - kTileBias - s_rng[1];
        const int z = (int)(klo[k] & 0xfffff) - kTileBias - s_rng[2];
        pk[k] = ((g * R[0] + x) * R[1] + y) * R[2] + z;
        atomicOr((unsigned long long*)&s_bits[pk[k] >> 6], 1ull << (pk[k] & 63));
      }
      __syncthreads();
      int nt;
      const int wex = block_excl_scan<int, kTilesThreads>(tid < nw ? popc64(s_bits[tid]) : 0, s_wave, nt);
      if (tid < nw) s_wpre[tid] = wex;
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kTilesItems; ++k) {
        if (pk[k] < 0) continue;
        const int w = pk[k] >> 6;
        const int t = s_wpre[w] + popc64(s_bits[w] & ((1ull << (pk[k] & 63)) - 1));
        tile_of_cand[tid * kTilesItems + k] = t;
        utile[t] = make_int4((int32_t)((klo[k] >> 40) & 0xfffff) - kTileBias,
                             (int32_t)((klo[k] >> 20) & 0xfffff) - kTileBias, (int32_t)(klo[k] & 0xfffff) - kTileBias,
                             (int32_t)((khi[k] << 4) | (klo[k] >> 60)));
      }
      // grid g's tiles begin at the rank of its first point g * Rx * Ry * Rz
      const int per_grid = R[0] * R[1] * R[2];
      for (int g = tid; g <= B; g += kTilesThreads) {
        if (g == B) {
          grid_tile_begin[g] = nt;
        } else {
          const int q = g * per_grid;
          const int w = q >> 6;
          grid_tile_begin[g] = s_wpre[w] + popc64(s_bits[w] & ((1ull << (q & 63)) - 1));
        }
      }
      if (tid == 0) *d_num_tiles = nt;
      if (zero_child) {
        ulonglong2* tc = reinterpret_cast<ulonglong2*>(tile_child);
        for (i64 k = tid; k < (i64)nt * 256; k += kTilesThreads) tc[k] = make_ulonglong2(0, 0);
      }
      return;
    }
  }
  int rank = 0;  // thread tid < K: the rank of key tid, which it holds in rhi, rlo, rv
  u64 rhi = 0, rlo = 0;
  uint32_t rv = 0;
  // More than 64 and at most kTilesThreads keys: the compacted keys are grouped
  // by grid (candidates follow the source uppers, which are in grid order), so a
  // key's rank is the first index of its grid's run plus its rank inside the
  // run. The run bounds come from two binary searches over the keys' grids;
  // when no run holds more than kSegMax keys, each thread ranks its key against
  // its own run only (a few keys per grid on large batches of small members).
  bool ranked = false;  // uniform
  if (K > kWave && K <= kTilesThreads) {
    __syncthreads();
    auto grid_at = [&](int i) { return (int32_t)((s_hi[i] << 4) | (s_lo[i] >> 60)); };
    int lo_b = 0, hi_b = 0;
    if (tid < K) {
      const int32_t g = grid_at(tid);
      int a = 0, b = tid;  // first index of grid g: in [0, tid]
      while (a < b) {
        const int mid = (a + b) >> 1;
        if (grid_at(mid) < g) a = mid + 1; else b = mid;
      }
      lo_b = a;
      a = tid + 1;
      b = K;  // one past its last index: in [tid + 1, K]
      while (a < b) {
        const int mid = (a + b) >> 1;
        if (grid_at(mid) <= g) a = mid + 1; else b = mid;
      }
      hi_b = a;
    }
    const int mseg = wave_max_i32(hi_b - lo_b);
    if (lane == 0) s_wave[wv] = mseg;
    __syncthreads();
    int mx = 0;
#pragma unroll
    for (int w = 0; w < kTilesThreads / kWave; ++w) mx = max(mx, s_wave[w]);
    __syncthreads();  // s_wave is free again
    if (mx <= kSegMax) {
      ranked = true;
      if (tid < K) {
        rhi = s_hi[tid];
        rlo = s_lo[tid];
        rv = s_v[tid];
        int c = 0;
        for (int j = lo_b; j < hi_b; ++j) {
          const u64 oh = s_hi[j], ol = s_lo[j];
          const uint32_t ov = s_v[j];
          c += (oh != rhi ? oh < rhi : (ol != rlo ? ol < rlo : ov < rv)) ? 1 : 0;
        }
        rank = lo_b + c;
      }
      // place every key at its rank, in place, then the head flags below
      __syncthreads();
      if (tid < K) {
        s_hi[rank] = rhi;
        s_lo[rank] = rlo;
        s_v[rank] = rv;
      }
      __syncthreads();
    }
  }
  // Up to kRankMax keys: a rank sort (keys are distinct through their candidate
  // index). With Kp = K rounded up to a power of two (>= 64), T = 1024 / Kp
  // threads share each key: thread (part, i) counts the keys smaller than key i
  // among its 1/T of the keys; the partial ranks meet in LDS.
  int32_t* s_cnt = reinterpret_cast<int32_t*>(lds + kTL_cnt);
  if (!ranked && K <= kRankMax) {
    int Kp = kWave;
    while (Kp < K) Kp <<= 1;
    const int T = kTilesThreads / Kp;
    const int ki = tid % Kp, part = tid / Kp;
    const int per = (K + T - 1) / T;
    __syncthreads();
    {
      int c = 0;
      if (ki < K) {
        const u64 hi = s_hi[ki], lo = s_lo[ki];
        const uint32_t v = s_v[ki];
        const int j1 = min(K, (part + 1) * per);
        for (int j = part * per; j < j1; ++j) {
          const u64 oh = s_hi[j], ol = s_lo[j];
          const uint32_t ov = s_v[j];
          c += (oh != hi ? oh < hi : (ol != lo ? ol < lo : ov < v)) ? 1 : 0;
        }
      }
      s_cnt[part * Kp + ki] = c;
    }
    __syncthreads();
    if (tid < K) {
      for (int q = 0; q < T; ++q) rank += s_cnt[q * Kp + tid];
      rhi = s_hi[tid];
      rlo = s_lo[tid];
      rv = s_v[tid];
    }
    if (K > kWave) {
      // place every key at its rank, in place (all keys are in registers first),
      // then the block-wide head flags below
      __syncthreads();
      if (tid < K) {
        s_hi[rank] = rhi;
        s_lo[rank] = rlo;
        s_v[rank] = rv;
      }
      __syncthreads();
    }
  }
  if (K <= kWave) {
    // at most 64 keys: wave 0 places them at their ranks (LDS, past the first
    // kWave entries), reads them back sorted, deduplicates and scatters with no
    // further block barrier
    if (wv == 0) {
      if (lane < K) {
        s_hi[kWave + rank] = rhi;
        s_lo[kWave + rank] = rlo;
        s_v[kWave + rank] = rv;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const u64 hi = lane < K ? s_hi[kWave + lane] : ~0ull, lo = lane < K ? s_lo[kWave + lane] : ~0ull;
      const uint32_t v = lane < K ? s_v[kWave + lane] : 0xffffffffu;
      const u64 ph = __shfl_up(hi, 1, kWave), pl = __shfl_up(lo, 1, kWave);
      const int head = lane < K && (lane == 0 || !(ph == hi && pl == lo)) ? 1 : 0;
      const int inc = wave_incl_scan(head);
      const int nt = __shfl(inc, kWave - 1, kWave);
      const int32_t g = (int32_t)((hi << 4) | (lo >> 60));  // grid of this lane's key
      const int32_t gp = __shfl_up(g, 1, kWave);
      if (lane < K) {
        const int t = inc - 1;
        if (v < (uint32_t)n) tile_of_cand[v] = t;
        if (head) {
          utile[t] = make_int4((int32_t)((lo >> 40) & 0xfffff) - kTileBias, (int32_t)((lo >> 20) & 0xfffff) - kTileBias,
                               (int32_t)(lo & 0xfffff) - kTileBias, g);
          for (int q = (lane == 0 ? -1 : gp) + 1; q <= g; ++q) grid_tile_begin[q] = t;
          if (t == nt - 1)
            for (int q = g + 1; q <= B; ++q) grid_tile_begin[q] = nt;
        }
      }
      if (nt == 0)
        for (int q = lane; q <= B; q += kWave) grid_tile_begin[q] = 0;
      if (lane == 0) {
        *d_num_tiles = nt;
        s_nt = nt;
      }
    }
    __syncthreads();
    if (zero_child) {
      ulonglong2* tc = reinterpret_cast<ulonglong2*>(tile_child);
      for (i64 k = tid; k < (i64)s_nt * 256; k += kTilesThreads) tc[k] = make_ulonglong2(0, 0);
    }
    return;
  }
  if (!ranked && K > kRankMax) {  // LDS bitonic sort
    int P = 2;
    while (P < K) P <<= 1;
    if (K <= kTilesThreads) {
      // one key per thread: stages whose partner is in the same wave exchange with
      // shuffles, only the wider ones go through LDS
      __syncthreads();
      u64 hi = tid < K ? s_hi[tid] : ~0ull, lo = tid < K ? s_lo[tid] : ~0ull;  // padding sorts last
      uint32_t v = tid < K ? s_v[tid] : 0xffffffffu;
      const bool act = tid < P;  // whole waves: P is a power of two >= 128
      for (int k = 2; k <= P; k <<= 1) {
        for (int jj = k >> 1; jj > 0; jj >>= 1) {
          u64 oh = 0, ol = 0;
          uint32_t ov = 0;
          if (jj >= kWave) {  // uniform
            __syncthreads();
            if (act) {
              s_hi[tid] = hi;
              s_lo[tid] = lo;
              s_v[tid] = v;
            }
            __syncthreads();
            if (act) {
              oh = s_hi[tid ^ jj];
              ol = s_lo[tid ^ jj];
              ov = s_v[tid ^ jj];
            }
          } else if (act) {
            oh = __shfl_xor(hi, jj, kWave);
            ol = __shfl_xor(lo, jj, kWave);
            ov = (uint32_t)__shfl_xor((int)v, jj, kWave);
          }
          if (!act) continue;
          const bool gt = hi != oh ? hi > oh : (lo != ol ? lo > ol : v > ov);
          const bool lt = hi != oh ? hi < oh : (lo != ol ? lo < ol : v < ov);
          const bool up = (tid & k) == 0, lower = (tid & jj) == 0;
          if (up ? (lower ? gt : lt) : (lower ? lt : gt)) {
            hi = oh;
            lo = ol;
            v = ov;
          }
        }
      }
      __syncthreads();
      if (act) {
        s_hi[tid] = hi;
        s_lo[tid] = lo;
        s_v[tid] = v;
      }
      __syncthreads();
    } else {
      for (int i = K + tid; i < P; i += kTilesThreads) {  // padding sorts last
        s_hi[i] = ~0ull;
        s_lo[i] = ~0ull;
        s_v[i] = 0xffffffffu;
      }
      __syncthreads();
      for (int k = 2; k <= P; k <<= 1) {
        for (int jj = k >> 1; jj > 0; jj >>= 1) {
          for (int i = tid; i < P; i += kTilesThreads) {
            const int ixj = i ^ jj;
            if (ixj > i) {
              const bool up = (i & k) == 0;
              const u64 ah = s_hi[i], al = s_lo[i], bh = s_hi[ixj], bl = s_lo[ixj];
              const uint32_t av = s_v[i], bv = s_v[ixj];
              const bool gt = ah != bh ? ah > bh : (al != bl ? al > bl : av > bv);
              if (gt == up) {
                s_hi[i] = bh;
                s_lo[i] = bl;
                s_v[i] = bv;
                s_hi[ixj] = ah;
                s_lo[ixj] = al;
                s_v[ixj] = av;
              }
            }
          }
          __syncthreads();
        }
      }
    }
  }
  // heads among the K sorted keys and their exclusive scan (blocked again)
  int f[kTilesItems];
  int sum = 0;
#pragma unroll
  for (int k = 0; k < kTilesItems; ++k) {
    const int i = tid * kTilesItems + k;
    f[k] = i < K && (i == 0 || !(s_hi[i] == s_hi[i - 1] && s_lo[i] == s_lo[i - 1])) ? 1 : 0;
    sum += f[k];
  }
  int total;
  int ex = block_excl_scan<int, kTilesThreads>(sum, s_wave, total);
#pragma unroll
  for (int k = 0; k < kTilesItems; ++k) {
    const int i = tid * kTilesItems + k;
    ex += f[k];
    if (i < K) {
      const uint32_t v = s_v[i];
      const int t = ex - 1;
      if (v < (uint32_t)n) tile_of_cand[v] = t;
      if (f[k]) {
        const u64 kh = s_hi[i], kl = s_lo[i];
        const int32_t g = (int32_t)((kh << 4) | (kl >> 60));
        utile[t] = make_int4((int32_t)((kl >> 40) & 0xfffff) - kTileBias, (int32_t)((kl >> 20) & 0xfffff) - kTileBias,
                             (int32_t)(kl & 0xfffff) - kTileBias, g);
        s_g[t] = g;
      }
    }
  }
  if (tid == 0) *d_num_tiles = total;
  __syncthreads();
  const int nt = total;
  if (nt == 0) {
    for (int g = tid; g <= B; g += kTilesThreads) grid_tile_begin[g] = 0;
  } else {
    for (int t = tid; t < nt; t += kTilesThreads) {
      const int g = s_g[t];
      const int gp = t == 0 ? -1 : s_g[t - 1];
      for (int q = gp + 1; q <= g; ++q) grid_tile_begin[q] = t;
      if (t == nt - 1)
        for (int q = g + 1; q <= B; ++q) grid_tile_begin[q] = nt;
    }
  }
  if (zero_child) {
    ulonglong2* tc = reinterpret_cast<ulonglong2*>(tile_child);
    for (i64 k = tid; k < (i64)nt * 256; k += kTilesThreads) tc[k] = make_ulonglong2(0, 0);
  }
}

__global__ void __launch_bounds__(kTilesThreads) k_tiles_small(const int4* upper_origin, const u64* upper_mask,
                                                               int32_t n_upper, int op, int m, int32_t B,
                                                               int4* utile, int32_t* tile_of_cand,
                                                               int32_t* d_num_tiles, int32_t* grid_tile_begin,
                                                               u64* tile_child, int zero_child,
                                                               const uint32_t* upper_reach, int32_t* readback,
                                                               const int32_t* src_status, int32_t* zero_word) {
  __shared__ __align__(16) char lds[kTilesLds];
  if (zero_word && threadIdx.x == 0) *zero_word = 0;
  tiles_small_body(upper_origin, upper_mask, n_upper, op, m, B, utile, tile_of_cand, d_num_tiles, grid_tile_begin,
                   tile_child, zero_child, upper_reach, readback, src_status, lds);
}

// ------------------------------------------------------------------ stage: lowers
// Target lower of source lower K for candidate j, and the index (among the
// parent upper's tile candidates) of the tile that holds it.
struct LowerTarget {
  I3 k;
  int jt;
  bool ok;
};

__device__ __forceinline__ LowerTarget lower_target(const int4 o, int j, int op) {
  const i64 kx = o.x >> 7, ky = o.y >> 7, kz = o.z >> 7;
  LowerTarget r;
  if (op == TC_OP_REFINE) {
    const I3 q = octant(j);
    r.k = {2 * kx + q.x, 2 * ky + q.y, 2 * kz + q.z};
    r.jt = octant_index((r.k.x >> 5) - 2 * (kx >> 5), (r.k.y >> 5) - 2 * (ky >> 5), (r.k.z >> 5) - 2 * (kz >> 5));
  } else if (op == TC_OP_COARSEN) {
    r.k = {kx >> 1, ky >> 1, kz >> 1};
    r.jt = 0;
  } else {
    const I3 e = box_offset(j, op);
    r.k = {kx + e.x, ky + e.y, kz + e.z};
    r.jt = box_index((r.k.x >> 5) - (kx >> 5), (r.k.y >> 5) - (ky >> 5), (r.k.z >> 5) - (kz >> 5), op);
  }
  r.ok = lower_ok(r.k.x) && lower_ok(r.k.y) && lower_ok(r.k.z);
  return r;
}

__device__ __forceinline__ int upper_child_bit(const I3& k) {
  return (int)((((k.x & 31) * 32) + (k.y & 31)) * 32 + (k.z & 31));
}

// Pair i = (source lower l, candidate j) sets its target lower's bit in the
// target tile's 32^3 candidate mask.
// `reach` (when non-null) holds every source lower's reach set, replacing the
// per-pair mask scan of lower_reaches.
__device__ __forceinline__ bool pair_reaches(const u64* lower_mask, const uint32_t* reach, i64 l, int op, int j) {
  if (op == TC_OP_COARSEN) return true;
  return reach ? ((reach[l] >> j) & 1u) != 0 : lower_reaches(lower_mask + l * 64, op, j);
}

__device__ __forceinline__ void lower_mark_one(i64 i, const int4* lower_origin, const u64* lower_mask,
                                               const uint32_t* reach, int op, int m, const int32_t* tile_of_cand,
                                               int32_t num_tiles, u64* tile_child, int32_t* flags) {
  const i64 l = i / m;
  const int j = (int)(i % m);
  const int4 o = lower_origin[l];
  const LowerTarget tg = lower_target(o, j, op);
  if (!tg.ok || !pair_reaches(lower_mask, reach, l, op, j)) return;
  const int32_t t = tile_of_cand[(i64)o.w * m + tg.jt];
  if (t < 0 || t >= num_tiles) {
    set_flag(flags, kFlagInternal);
    return;
  }
  const int bit = upper_child_bit(tg.k);
  atomicOr((unsigned long long*)&tile_child[(i64)t * 512 + (bit >> 6)], 1ull << (bit & 63));
}

// Pair i = (l, j): the candidate index of its target (its rank in the tile's
// mask, after the tile's base), the candidate's origin, and the candidate ->
// source table entry of l.
__device__ __forceinline__ void lower_nbr_one(i64 i, const int4* lower_origin, const u64* lower_mask,
                                              const uint32_t* reach, int op, int m, int m_src,
                                              const int32_t* tile_of_cand, const u64* tile_child,
                                              const uint16_t* tile_prefix, const int32_t* tile_lower_base,
                                              int32_t num_tiles, int32_t num_cands, int32_t* lower_nbr,
                                              int4* cand_origin, int32_t* cand_src, int32_t* flags) {
  const i64 l = i / m;
  const int j = (int)(i % m);
  const int4 o = lower_origin[l];
  const LowerTarget tg = lower_target(o, j, op);
  if (!tg.ok || !pair_reaches(lower_mask, reach, l, op, j)) {
    lower_nbr[i] = -1;
    return;
  }
  const int32_t t = tile_of_cand[(i64)o.w * m + tg.jt];
  if (t < 0 || t >= num_tiles) {
    lower_nbr[i] = -1;
    set_flag(flags, kFlagInternal);
    return;
  }
  const int bit = upper_child_bit(tg.k);
  const int w = bit >> 6, b = bit & 63;
  const u64 word = tile_child[(i64)t * 512 + w];
  const int32_t c = tile_lower_base[t] + tile_prefix[(i64)t * 512 + w] + popc64(word & ((1ull << b) - 1));
  if (!((word >> b) & 1ull) || c < 0 || c >= num_cands) {
    lower_nbr[i] = -1;
    set_flag(flags, kFlagInternal);
    return;
  }
  lower_nbr[i] = c;
  cand_origin[c] = make_int4((int32_t)(tg.k.x * 128), (int32_t)(tg.k.y * 128), (int32_t)(tg.k.z * 128), t);
  int js;
  if (op == TC_OP_REFINE) {
    js = 0;
  } else if (op == TC_OP_COARSEN) {
    js = octant_index((o.x >> 7) & 1, (o.y >> 7) & 1, (o.z >> 7) & 1);
  } else {
    const I3 e = box_offset(j, op);
    js = index27(-e.x, -e.y, -e.z);
  }
  cand_src[(i64)c * m_src + js] = (int32_t)l;
}

__global__ void __launch_bounds__(256) k_lower_mark(const int4* lower_origin, const u64* lower_mask,
                                                    const uint32_t* reach, i64 n, int op, int m,
                                                    const int32_t* tile_of_cand, const int32_t* d_num_tiles,
                                                    u64* tile_child, int32_t* flags) {
  const i64 i = (i64)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  lower_mark_one(i, lower_origin, lower_mask, reach, op, m, tile_of_cand, *d_num_tiles, tile_child, flags);
}

__global__ void __launch_bounds__(256) k_lower_nbr(const int4* lower_origin, const u64* lower_mask,
                                                   const uint32_t* reach, i64 n, int op,
                                                   int m, int m_src, const int32_t* tile_of_cand,
                                                   const u64* tile_child, const uint16_t* tile_prefix,
                                                   const int32_t* tile_lower_base, const int32_t* d_num_tiles,
                                                   const int32_t* d_num_cands, int32_t* lower_nbr, int4* cand_origin,
                                                   int32_t* cand_src, int32_t* flags) {
  const i64 i = (i64)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  lower_nbr_one(i, lower_origin, lower_mask, reach, op, m, m_src, tile_of_cand, tile_child, tile_prefix,
                tile_lower_base, *d_num_tiles, *d_num_cands, lower_nbr, cand_origin, cand_src, flags);
}

// Small batches (at least one and at most kLowersSmallMax (lower, candidate)
// pairs, at most kLowersSmallTiles tile candidates): the whole lower stage in
// one workgroup:
// every source lower's reach set, marking, per-tile popcount prefix tables, the
// scan over tiles (candidate numbering), the empty candidate -> source table,
// and the candidate indices / origins / sources. When the unique tiles are few
// (at most kLdsTiles, known only here) their candidate masks, prefix tables and
// bases live in LDS and the masks are copied out at the end; otherwise the same
// steps run on the global arrays; a block barrier orders what other waves wrote
// before a later phase reads it. Each thread owns two pairs, whose origins and tile
// indices are loaded once, up front, all in flight together. Replaces five
// launches of the general path.
constexpr int kLowersSmallMax = 2048;  // beyond this the five-launch path is faster
constexpr int kLowersSmallTiles = 1024;
constexpr int kLowersThreads = 1024;
constexpr int kLowersItems = kLowersSmallMax / kLowersThreads;
constexpr int kLdsTiles = 28;
constexpr int kReachMax = 512;  // source lowers with a reach set: n / m for m >= 8
static_assert(kReachMax <= kLowersThreads, "one given reach set per thread");

constexpr int kLL_tile = 0;
constexpr int kLL_tpre = kLL_tile + 8 * kLdsTiles * 512;
constexpr int kLL_base = kLL_tpre + 2 * kLdsTiles * 512;
constexpr int kLL_reach = kLL_base + 4 * ((kLowersSmallTiles + 4) / 4 * 4);
constexpr int kLL_wave = kLL_reach + 4 * kReachMax;
constexpr int kLowersLds = kLL_wave + 4 * (kLowersThreads / kWave);

__device__ __forceinline__ void lowers_small_body(
    const int4* lower_origin, const u64* lower_mask, i64 n, int op, int m, int m_src, const int32_t* tile_of_cand,
    const int32_t* d_num_tiles, u64* tile_child, uint16_t* tile_prefix, int32_t* tile_lower_base,
    int32_t* d_num_cands, u64* cand_child, int zero_cand_child, int32_t* lower_nbr, int4* cand_origin,
    int32_t* cand_src, int32_t* flags, const uint32_t* lower_reach, const int4 (&po)[kLowersItems],
    uint32_t reach_pre, char* lds) {
  u64* s_tile = reinterpret_cast<u64*>(lds + kLL_tile);
  uint16_t* s_tpre = reinterpret_cast<uint16_t*>(lds + kLL_tpre);
  int32_t* s_base = reinterpret_cast<int32_t*>(lds + kLL_base);
  uint32_t* s_reach = reinterpret_cast<uint32_t*>(lds + kLL_reach);
  int32_t* s_wave = reinterpret_cast<int32_t*>(lds + kLL_wave);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  constexpr int kWaves = kLowersThreads / kWave;
  const int32_t nt = *d_num_tiles;
  const i64 n_lower = n / m;
  // po: the origins of this thread's pairs (pair tid + k * kLowersThreads, clamped), loaded by the caller
  // reach set of every source lower: given (k_box_reach; thread l loaded lower l's
  // set, reach_pre), or one wave per lower, one mask word per lane, four lowers
  // per wave in flight
  if (lower_reach) {
    if (tid < n_lower) s_reach[tid] = reach_pre;
  } else if (op != TC_OP_COARSEN) {
    constexpr int kPer = 4;
    for (i64 l0 = wv * kPer; l0 < n_lower; l0 += kWaves * kPer) {
      u64 w4[kPer];
#pragma unroll
      for (int v = 0; v < kPer; ++v) w4[v] = lower_mask[min(l0 + v, n_lower - 1) * 64 + lane];
#pragma unroll
      for (int v = 0; v < kPer; ++v) {
        uint32_t code = lower_word_reach(w4[v], lane, op);
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) code |= (uint32_t)__shfl_xor((int)code, d, kWave);
        if (lane == 0 && l0 + v < n_lower) s_reach[l0 + v] = op == TC_OP_REFINE ? code : box_code_for_op(code, op, m);
      }
    }
  }
  const bool in_lds = nt <= kLdsTiles;  // uniform
  u64* tch = in_lds ? s_tile : tile_child;
  if (in_lds) {
    for (int k = tid; k < nt * 512; k += kLowersThreads) s_tile[k] = 0;
  } else {
    ulonglong2* tc2 = reinterpret_cast<ulonglong2*>(tile_child);
    for (i64 k = tid; k < (i64)nt * 256; k += kLowersThreads) tc2[k] = make_ulonglong2(0, 0);
  }
  // the barrier orders every wave's global stores before the other waves'
  // accesses after it (workgroup scope; nothing here is read by another workgroup)
  __syncthreads();
  // targets of the thread's pairs and their tiles
  LowerTarget tg[kLowersItems];
  int32_t tt[kLowersItems];
  bool act[kLowersItems];
#pragma unroll
  for (int k = 0; k < kLowersItems; ++k) {
    const i64 i = tid + k * kLowersThreads;
    const i64 ic = min(i, n - 1);
    const i64 l = ic / m;
    const int j = (int)(ic % m);
    tg[k] = lower_target(po[k], j, op);
    act[k] = i < n && tg[k].ok && (op == TC_OP_COARSEN || ((s_reach[l] >> j) & 1u) != 0);
  }
#pragma unroll
  for (int k = 0; k < kLowersItems; ++k) tt[k] = tile_of_cand[act[k] ? (i64)po[k].w * m + tg[k].jt : 0];
#pragma unroll
  for (int k = 0; k < kLowersItems; ++k) {
    if (!act[k]) continue;
    if (tt[k] < 0 || tt[k] >= nt) {
      set_flag(flags, kFlagInternal);
      continue;
    }
    const int bit = upper_child_bit(tg[k].k);
    atomicOr((unsigned long long*)&tch[(i64)tt[k] * 512 + (bit >> 6)], 1ull << (bit & 63));
  }
  __syncthreads();
  // per-tile prefix tables: one wave per tile, 8 words per lane
  for (int t = wv; t < nt; t += kWaves) {
    u64 wd[8];
    int sum = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      wd[k] = tch[(i64)t * 512 + lane * 8 + k];
      sum += popc64(wd[k]);
    }
    const int inc = wave_incl_scan(sum);
    int ex = inc - sum;
    uint32_t pk[4];  // the lane's 8 prefixes as 16-bit pairs: one 16-byte store
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e0 = ex;
      ex += popc64(wd[2 * k]);
      pk[k] = (uint32_t)e0 | ((uint32_t)ex << 16);
      ex += popc64(wd[2 * k + 1]);
    }
    const uint4 pv = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    reinterpret_cast<uint4*>(tile_prefix)[(i64)t * 64 + lane] = pv;
    if (in_lds) reinterpret_cast<uint4*>(s_tpre)[t * 64 + lane] = pv;
    if (lane == kWave - 1) s_base[t] = inc;
  }
  __syncthreads();
  // candidate numbering: exclusive scan of the tiles' counts (one per thread)
  const int cnt = tid < nt ? s_base[tid] : 0;
  int total;
  const int ex = block_excl_scan<int, kLowersThreads>(cnt, s_wave, total);
  if (tid < nt) {
    s_base[tid] = ex;
    tile_lower_base[tid] = ex;
  }
  if (tid == 0) {
    s_base[nt] = total;
    tile_lower_base[nt] = total;
    *d_num_cands = total;
  }
  for (i64 k = tid; k < (i64)total * m_src; k += kLowersThreads) cand_src[k] = -1;
  if (zero_cand_child)
    for (i64 k = tid; k < (i64)total * 64; k += kLowersThreads) cand_child[k] = 0;
  __syncthreads();  // the fills land before other waves' table entries below
  // candidate index of every pair, its origin and its candidate -> source entry
#pragma unroll
  for (int k = 0; k < kLowersItems; ++k) {
    const i64 i = tid + k * kLowersThreads;
    if (i >= n) break;
    if (!act[k] || tt[k] < 0 || tt[k] >= nt) {
      lower_nbr[i] = -1;
      continue;
    }
    const int t = tt[k];
    const int bit = upper_child_bit(tg[k].k);
    const int w = bit >> 6, b = bit & 63;
    const u64 word = tch[(i64)t * 512 + w];
    const int pre = in_lds ? s_tpre[t * 512 + w] : tile_prefix[(i64)t * 512 + w];
    const int32_t c = s_base[t] + pre + popc64(word & ((1ull << b) - 1));
    if (!((word >> b) & 1ull) || c < 0 || c >= total) {
      lower_nbr[i] = -1;
      set_flag(flags, kFlagInternal);
      continue;
    }
    const int4 o = po[k];
    const i64 l = i / m;
    lower_nbr[i] = c;
    cand_origin[c] = make_int4((int32_t)(tg[k].k.x * 128), (int32_t)(tg[k].k.y * 128), (int32_t)(tg[k].k.z * 128), t);
    int js;
    if (op == TC_OP_REFINE) {
      js = 0;
    } else if (op == TC_OP_COARSEN) {
      js = octant_index((o.x >> 7) & 1, (o.y >> 7) & 1, (o.z >> 7) & 1);
    } else {
      const I3 e = box_offset((int)(i % m), op);
      js = index27(-e.x, -e.y, -e.z);
    }
    cand_src[(i64)c * m_src + js] = (int32_t)l;
  }
  if (in_lds) {  // the node writers read the masks later
    const ulonglong2* src2 = reinterpret_cast<const ulonglong2*>(s_tile);
    ulonglong2* dst2 = reinterpret_cast<ulonglong2*>(tile_child);
    for (int k = tid; k < nt * 256; k += kLowersThreads) dst2[k] = src2[k];
  }
}

// Tile and lower stages of a small batch in one workgroup: the tile stage's
// results reach the lower stage through global memory written and read by this
// workgroup (ordered by the block barrier between them), and both stages carve
// their LDS from the same block.
constexpr int kNodesLds = kTilesLds > kLowersLds ? kTilesLds : kLowersLds;
static_assert(kTilesThreads == kLowersThreads, "one workgroup shape for both stages");
__global__ void __launch_bounds__(kTilesThreads) k_nodes_small(
    const int4* upper_origin, const u64* upper_mask, int32_t n_upper, int32_t B, int4* utile,
    int32_t* grid_tile_begin, const uint32_t* upper_reach, int32_t* readback, const int32_t* src_status,
    const int4* lower_origin, const u64* lower_mask, i64 n, int op, int m, int m_src, int32_t* tile_of_cand,
    int32_t* d_num_tiles, u64* tile_child, uint16_t* tile_prefix, int32_t* tile_lower_base, int32_t* d_num_cands,
    u64* cand_child, int32_t* lower_nbr, int4* cand_origin, int32_t* cand_src, const uint32_t* lower_reach) {
  __shared__ __align__(16) char lds[kNodesLds];
  // the lower stage's first loads (its pairs' origins, the given reach sets)
  // go out with the tile stage's (n >= 1; clamped indices)
  int4 po[kLowersItems];
#pragma unroll
  for (int k = 0; k < kLowersItems; ++k)
    po[k] = lower_origin[min((i64)(threadIdx.x + k * kLowersThreads), n - 1) / m];
  const uint32_t reach_pre = lower_reach ? lower_reach[min((i64)threadIdx.x, n / m - 1)] : 0u;
  tiles_small_body(upper_origin, upper_mask, n_upper, op, m, B, utile, tile_of_cand, d_num_tiles, grid_tile_begin,
                   tile_child, 0, upper_reach, readback, src_status, lds);
  __syncthreads();
  lowers_small_body(lower_origin, lower_mask, n, op, m, m_src, tile_of_cand, d_num_tiles, tile_child, tile_prefix,
                    tile_lower_base, d_num_cands, cand_child, 0, lower_nbr, cand_origin, cand_src, readback,
                    lower_reach, po, reach_pre, lds);
}

// ------------------------------------------------------------------ stage: leaves (marking)
// Refine: the 4^3 sub-block q of the source leaf becomes child leaf q.
__device__ __forceinline__ bool subblock_nonempty(const u64 W[8], const I3& q) {
  const u64 xs = q.x ? (W[4] | W[5] | W[6] | W[7]) : (W[0] | W[1] | W[2] | W[3]);
  const u64 ym = q.y ? 0xffffffff00000000ull : 0x00000000ffffffffull;
  const u64 zm = q.z ? 0xf0f0f0f0f0f0f0f0ull : 0x0f0f0f0f0f0f0f0full;
  return (xs & ym & zm) != 0;
}

// Leaf marking: refine from the source side (a target lower has exactly one
// source lower, so its mask is stored whole, no zero fill), coarsen and the box
// ops from the target side (below).

// Refine: two workgroups per source lower, one per half along x (the leaves
// with local x < 8 come first in x-major order, so each half is a contiguous
// range of leaves, and its children land in the 4 target lowers of that x
// octant only). A workgroup marks, in LDS copies of its 4 target lowers' 16^3
// masks, the non-empty 2^3 sub-blocks of its leaves; each target lower has this
// one source, so the workgroup stores the whole masks with their prefixes and
// counts (wave v: target 4h + v). Halving the lower keeps the largest
// workgroups short.
__global__ void __launch_bounds__(256) k_leaf_mark_lower(const int4* leaf_origin, const u64* leaf_mask,
                                                         const int32_t* lower_first, const u64* lower_mask,
                                                         const uint16_t* lower_prefix, int op, int m,
                                                         const int32_t* lower_nbr, const int32_t* d_num_cands,
                                                         u64* cand_child, uint16_t* cand_prefix,
                                                         i64* cand_counts, int32_t* flags) {
  constexpr int kPer = 1;  // leaves per thread per batch
  __shared__ unsigned long long s_mask[4 * 64];
  const i64 l = blockIdx.x >> 1;
  const int h = (int)(blockIdx.x & 1);
  const int wv = threadIdx.x / kWave;
  // loads indexed by the lower alone, first: its leaf range (words 0..31 hold
  // x < 8) and the candidate its wave's target lower became
  const i64 first0 = lower_first[l];
  const int half = lower_prefix[l * 64 + 32];  // leaves with x < 8
  const int total = lower_prefix[l * 64 + 63] + popc64(lower_mask[l * 64 + 63]);
  const int32_t ncand = *d_num_cands;
  const int32_t nbr = lower_nbr[l * m + 4 * h + wv];  // m == 8
  s_mask[threadIdx.x] = 0;
  const i64 first = first0 + (h ? half : 0);
  const int count = h ? total - half : half;
  __syncthreads();
  // leaves kPer * 256 at a time, the next batch's loads issued before this
  // batch is marked (half a dense lower has up to 2048 leaves)
  int4 o[kPer];
  u64 W[kPer][8];
  auto load_batch = [&](int k0) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {  // clamped: every leaf of the batch in flight together
      const i64 i = first + max(0, min(k0 + u * 256 + (int)threadIdx.x, count - 1));
      o[u] = leaf_origin[i];
#pragma unroll
      for (int q = 0; q < 8; ++q) W[u][q] = leaf_mask[i * 8 + q];
    }
  };
  if (count > 0) load_batch(0);
  for (int k0 = 0; k0 < count; k0 += kPer * 256) {
    int4 oc[kPer];
    u64 Wc[kPer][8];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      oc[u] = o[u];
#pragma unroll
      for (int q = 0; q < 8; ++q) Wc[u][q] = W[u][q];
    }
    if (k0 + kPer * 256 < count) load_batch(k0 + kPer * 256);
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      if (k0 + u * 256 + (int)threadIdx.x >= count) continue;
      const i64 mx = oc[u].x >> 3, my = oc[u].y >> 3, mz = oc[u].z >> 3;  // leaf coordinates
      const i64 lx = mx & 15, ly = my & 15, lz = mz & 15;              // position inside the lower
      if ((int)(lx >> 3) != h) {  // cannot happen for a consistent lower
        set_flag(flags, kFlagInternal);
        continue;
      }
      const int j = octant_index(0, ly >> 3, lz >> 3);  // all children share one target lower (4h + j)
#pragma unroll
      for (int qx = 0; qx < 2; ++qx) {
        u64 word = 0;
        const i64 x = (2 * lx + qx) & 15;
#pragma unroll
        for (int qy = 0; qy < 2; ++qy)
#pragma unroll
          for (int qz = 0; qz < 2; ++qz) {
            const I3 q{qx, qy, qz};
            if (!subblock_nonempty(Wc[u], q)) continue;
            if (!leaf_ok(2 * mx + qx) || !leaf_ok(2 * my + qy) || !leaf_ok(2 * mz + qz)) {
              set_flag(flags, kFlagOverflow);
              continue;
            }
            word |= 1ull << ((((2 * ly + qy) & 3) * 16) + ((2 * lz + qz) & 15));
          }
        // children with this qx share the word x*4 + (y >> 2) of the target mask
        if (word) atomicOr(&s_mask[j * 64 + x * 4 + (((2 * ly) & 15) >> 2)], word);
      }
    }
  }
  __syncthreads();
  // wave v flushes target 4h + v (its 64 words)
  const u64 word = s_mask[threadIdx.x];
  if (nbr < 0 || nbr >= ncand) {  // uniform per wave
    if (word) set_flag(flags, kFlagInternal);  // a marked target must have a candidate
    return;
  }
  store_candidate(nbr, word, cand_child, cand_prefix, cand_counts);
}

// Coarsen: one wave per candidate lower T, pulling from the source lowers of its
// 8 octants (cand_src). Target leaf t = (tx, ty, tz) in [0,16)^3 holds a voxel
// exactly when one of the 2^3 source leaves 2(t & 7) + {0,1}^3 of the source
// lower in octant t >> 3 exists (a source leaf is never empty), so the target
// mask is the OR of 2x2x2 blocks of the source lowers' 16^3 masks; the leaves
// themselves are not read. Lane w builds target word w (x = w >> 2, rows
// y = 4 (w & 3) + r, every z) and the wave stores it with prefix and count.
__global__ void __launch_bounds__(256) k_mark_coarsen(const int32_t* cand_src, const int32_t* d_num_cands,
                                                      const u64* src_lower_mask, int32_t n_src_lower,
                                                      u64* cand_child, uint16_t* cand_prefix, i64* cand_counts,
                                                      int32_t* flags) {
  const i64 c = (i64)blockIdx.x * 4 + threadIdx.x / kWave;
  if (c >= *d_num_cands) return;  // uniform per wave
  const int w = threadIdx.x & (kWave - 1);
  const int tx = w >> 2, yq = w & 3;
  int32_t s[2];
  u64 lo_w[2][2], hi_w[2][2];  // [jz][a]: source rows 8(yq&1) .. +3 and +4 .. +7 of column 2(tx&7) + a
#pragma unroll
  for (int jz = 0; jz < 2; ++jz) {
    s[jz] = cand_src[c * 8 + octant_index(tx >> 3, yq >> 1, jz)];
    if (s[jz] >= n_src_lower) {
      set_flag(flags, kFlagInternal);
      s[jz] = -1;
    }
    const i64 ls = s[jz] >= 0 ? s[jz] : 0;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const i64 sw = ls * 64 + (2 * (tx & 7) + a) * 4 + 2 * (yq & 1);
      lo_w[jz][a] = src_lower_mask[sw];
      hi_w[jz][a] = src_lower_mask[sw + 1];
    }
  }
  u64 word = 0;
#pragma unroll
  for (int jz = 0; jz < 2; ++jz) {
    if (s[jz] < 0) continue;
    const u64 x0 = lo_w[jz][0] | lo_w[jz][1], x1 = hi_w[jz][0] | hi_w[jz][1];  // both source columns
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // source rows 2r and 2r + 1 of the 8: rows 0..3 in x0, 4..7 in x1 (16 bits per row)
      const u64 src = r < 2 ? x0 : x1;
      const int rr = (2 * r) & 3;
      uint32_t v = (uint32_t)((src >> (16 * rr)) | (src >> (16 * (rr + 1)))) & 0xffffu;
      v = (v | (v >> 1)) & 0x5555u;  // z pairs -> even bits
      v = (v | (v >> 1)) & 0x3333u;
      v = (v | (v >> 2)) & 0x0f0fu;
      v = (v | (v >> 4)) & 0x00ffu;  // 8 target z values
      word |= (u64)v << (16 * r + 8 * jz);
    }
  }
  store_candidate(c, word, cand_child, cand_prefix, cand_counts);
}

// ------------------------------------------------------------------ stage: leaves, box ops (pull)
// Box ops mark from the target side: one resident round of workgroups, each
// looping over its candidate lowers C (the next one's loads in flight). C's
// sources are the source lowers at C + d, d in {-1,0,1}^3; from the one at
// offset d only the leaves on the face / edge / corner that touches C can reach
// it (offset t = -d on each axis where d is non-zero). The workgroup stages the
// mask words that hold such leaves and a block scan of their counts in LDS;
// every thread then takes one leaf at a time (its word from an LDS map of the
// scan, or a binary search over it past the map), tests which offsets of the
// box spill voxels into C and ORs the target bits into an LDS copy of C's 16^3
// leaf mask, which is stored whole at the end: no device atomics on the masks
// and no zero fill.
constexpr int kPullItems = 27 * 64;  // (source slot, mask word) pairs

__host__ __device__ constexpr u64 face_word_mask(int js, int w, int lo, int hi) {
  const int dx = js / 9 - 1, dy = (js / 3) % 3 - 1, dz = js % 3 - 1;
  if ((dx != 0 && (-dx < lo || -dx > hi)) || (dy != 0 && (-dy < lo || -dy > hi)) ||
      (dz != 0 && (-dz < lo || -dz > hi)))
    return 0;
  const int x = w >> 2, yq = w & 3;
  if ((dx < 0 && x != 15) || (dx > 0 && x != 0)) return 0;
  u64 m = ~0ull;
  if (dy < 0) m = yq == 3 ? 0xffff000000000000ull : 0;  // y = 15
  else if (dy > 0) m = yq == 0 ? 0xffffull : 0;         // y = 0
  if (dz < 0) m &= 0x8000800080008000ull;               // z = 15
  else if (dz > 0) m &= 0x0001000100010001ull;          // z = 0
  return m;
}

// The live items of a box: the (slot, word) pairs whose word can hold a leaf
// facing the candidate (the whole centre lower, the boundary words or bits of
// the faces, fewer for edges and corners): 324 for [-1,1]^3, 170 for either pad,
// against 27 * 64. Built at compile time, slot-major.
constexpr int kLiveMax = 384;
constexpr int kLivePer = (kLiveMax + 255) / 256;  // per thread
struct PullTable {
  int n;
  uint16_t item[kLiveMax];  // js * 64 + w
};
constexpr PullTable make_pull_table(int lo, int hi) {
  PullTable t{};
  for (int it = 0; it < kPullItems; ++it)
    if (face_word_mask(it >> 6, it & 63, lo, hi) != 0 && t.n < kLiveMax) t.item[t.n++] = (uint16_t)it;
  return t;
}
__constant__ PullTable kPullDilate = make_pull_table(-1, 1);
__constant__ PullTable kPullNeg = make_pull_table(-1, 0);
__constant__ PullTable kPullPos = make_pull_table(0, 1);
static_assert(make_pull_table(-1, 1).n == 324 && make_pull_table(-1, 0).n == 170 && make_pull_table(0, 1).n == 170,
              "live pull items per box");

template <int lo, int hi>
__device__ __forceinline__ const PullTable& pull_table() {
  return lo < 0 && hi > 0 ? kPullDilate : (lo < 0 ? kPullNeg : kPullPos);
}

// Position in C's frame (-1 .. 16 per axis) packed as 3 x 5 bits of p + 1.
__device__ __forceinline__ uint32_t pack_pos(int px, int py, int pz) {
  return (uint32_t)(px + 1) | ((uint32_t)(py + 1) << 5) | ((uint32_t)(pz + 1) << 10);
}

// Marks the target leaves of C that a source leaf at `pos` (C's frame, packed
// by pack_pos) with mask words W spills voxels into: offset t of the box is
// marked when the leaf holds a voxel on each face t points across (x: word 0 or
// 7, y: row byte 0 or 7, z: bit 0 or 7 of the row bytes; t = 0 on an axis asks
// for any voxel). Per (tx, ty) the three z flags form a 3-bit pattern that is
// shifted into place (and clipped to the leaf row) at once.
__device__ __forceinline__ uint32_t z_pattern(uint32_t r) {  // r: the OR of the rows' bytes (8 bits)
  return (r & 1u) | (r != 0u ? 2u : 0u) | ((r >> 5) & 4u);  // tz = -1, 0, +1
}
__device__ __forceinline__ void mark_box_leaf(const u64 W[8], uint32_t pos, int lo, int hi,
                                              unsigned long long* s_mask) {
  const int px = (int)(pos & 31) - 1, py = (int)((pos >> 5) & 31) - 1, pz = (int)((pos >> 10) & 31) - 1;
  const u64 all = W[0] | W[1] | W[2] | W[3] | W[4] | W[5] | W[6] | W[7];
  // the z run of a pattern: bit k <-> target z = pz - 1 + k, kept inside [0, 15]
  const uint32_t zmask = lo < 0 ? 7u : 6u, zmask2 = hi > 0 ? 7u : 3u;  // taps the box holds
#pragma unroll
  for (int tx = lo; tx <= hi; ++tx) {
    const int qx = px + tx;
    const u64 xs = tx > 0 ? W[7] : (tx < 0 ? W[0] : all);  // voxels that spill toward tx
    const uint32_t xl = (uint32_t)xs, xh = (uint32_t)(xs >> 32);
    uint32_t fold = xl | xh;  // OR of the eight row bytes
    fold |= fold >> 16;
    fold |= fold >> 8;
#pragma unroll
    for (int ty = lo; ty <= hi; ++ty) {
      const int qy = py + ty;
      const uint32_t r = ty < 0 ? (xl & 0xffu) : (ty > 0 ? (xh >> 24) : (fold & 0xffu));  // row 0, row 7, any
      const uint32_t p3 = z_pattern(r) & zmask & zmask2;
      const uint32_t run = ((p3 << (pz + 1)) >> 2) & 0xffffu;  // bits of target z in 0..15
      if (!run || qx < 0 || qx > 15 || qy < 0 || qy > 15) continue;
      atomicOr(&s_mask[qx * 4 + (qy >> 2)], (unsigned long long)run << ((qy & 3) * 16));
    }
  }
}

constexpr int kMarkIlp = 1;  // leaves in flight per thread

// Erosion of a lower's 16^3 leaf mask by the box [lo, hi]^3, with positions
// outside the lower counted as set: bit p stays set when p + t is set or lies
// outside the lower for every t in the box. Lane w of one wave holds word w
// (x = w >> 2, rows y = 4 (w & 3) .. +3, bit (y & 3) * 16 + z); every lane of
// the wave must call it. The three axis passes run one after another (erosion
// by a box is erosion by its three axis segments in turn).
template <int lo, int hi>
__device__ __forceinline__ u64 erode_lower_mask(u64 m) {
  const int w = threadIdx.x & (kWave - 1);
  constexpr u64 kZ15 = 0x8000800080008000ull, kZ0s = 0x0001000100010001ull;  // z = 15 / z = 0 of each row
  u64 e = m;  // z: neighbours z + 1 (bit above) and z - 1 (bit below) inside the row
  if (hi > 0) e &= (m >> 1) | kZ15;
  if (lo < 0) e &= (m << 1) | kZ0s;
  // y: rows y + 1 / y - 1, across words for the rows at a word's edge
  const u64 up = (u64)__shfl_down((unsigned long long)e, 1, kWave);  // word w + 1
  const u64 dn = (u64)__shfl_up((unsigned long long)e, 1, kWave);    // word w - 1
  u64 f = e;
  if (hi > 0) f &= (e >> 16) | ((w & 3) < 3 ? up << 48 : 0xffff000000000000ull);
  if (lo < 0) f &= (e << 16) | ((w & 3) > 0 ? dn >> 48 : 0xffffull);
  // x: words w + 4 / w - 4
  const u64 xp = (u64)__shfl_down((unsigned long long)f, 4, kWave);
  const u64 xm = (u64)__shfl_up((unsigned long long)f, 4, kWave);
  u64 g = f;
  if (hi > 0) g &= (w >> 2) < 15 ? xp : ~0ull;
  if (lo < 0) g &= (w >> 2) > 0 ? xm : ~0ull;
  return g;
}

constexpr int kMarkMap = 4096;  // reaching leaves whose live item a workgroup maps in LDS (more: binary search)

template <int lo, int hi>  // the box [lo, hi]^3: dilate [-1, 1], pads [-1, 0] and [0, 1]
__global__ void __launch_bounds__(256) k_leaf_mark_box(const int32_t* cand_src, const int32_t* d_num_cands,
                                                       int32_t B, const tc_grid_header* src_headers,
                                                       const u64* src_lower_mask, const uint16_t* src_lower_prefix,
                                                       const int32_t* src_lower_first, const u64* src_leaf_mask,
                                                       int32_t n_src_lower, int32_t n_src_leaf, u64* cand_child,
                                                       uint16_t* cand_prefix, i64* cand_counts,
                                                       int32_t* flags) {
  const PullTable& tab = pull_table<lo, hi>();
  const int nlive = tab.n;
  __shared__ u64 s_word[kLiveMax];          // source mask word of each live item (unmasked)
  __shared__ int32_t s_base[kLiveMax];      // leaf index of the word's first leaf
  __shared__ int32_t s_excl[kLiveMax + 1];  // exclusive scan of the items' reaching leaves
  __shared__ uint16_t s_item[kLiveMax];     // js * 64 + w of each live item
  __shared__ unsigned long long s_mask[64];
  __shared__ u64 s_fm[kLiveMax];            // the item's mask of leaves to visit
  __shared__ u64 s_center[64];              // 16^3 mask of the co-located source lower
  __shared__ u64 s_skip[64];                // its leaves that spill onto marked positions only
  __shared__ uint16_t s_map[kMarkMap];      // live item of each reaching leaf
  __shared__ int32_t s_wave[256 / kWave];
  const int tid = threadIdx.x;
  // An output coordinate leaves int32 exactly when a grid's bbox, widened by
  // the box, does (its extreme voxels are present).
  if (blockIdx.x == 0) {
    for (int g = tid; g < B; g += 256) {
      const tc_grid_header h = src_headers[g];
      bool over = false;
      for (int a = 0; a < 3; ++a)
        over |= (i64)h.bbox_min[a] <= (i64)h.bbox_max[a] &&
                ((i64)h.bbox_min[a] + lo < INT32_MIN || (i64)h.bbox_max[a] + hi > INT32_MAX);
      if (over) set_flag(flags, kFlagOverflow);
    }
  }
  const i64 ncand = *d_num_cands;
  // Candidates: the workgroups of XCD x (workgroup b runs on XCD b % 8; the
  // launch is a multiple of 8 workgroups) take the x-th eighth of the
  // candidates, interleaved over that range, so neighbouring candidates, which
  // read the same source lowers and leaves, share one L2, and dense runs of
  // candidates spread over the XCD's workgroups.
  const int bpx = (int)(gridDim.x >> 3), xr = (int)(blockIdx.x & 7);
  const i64 c_end = ncand * (xr + 1) / 8;
  // this thread's live items (the same for every candidate)
  int item[kLivePer];
  u64 fm0[kLivePer];
#pragma unroll
  for (int k = 0; k < kLivePer; ++k) {
    const int li = tid * kLivePer + k;
    item[k] = tab.item[min(li, nlive - 1)];
    fm0[k] = li < nlive ? face_word_mask(item[k] >> 6, item[k] & 63, lo, hi) : 0;
  }
  // A candidate's staging loads in two levels, the next candidate's issued
  // while the current one is processed: its source lowers (slot 0 stands in for
  // an empty slot; n_src_lower >= 1 whenever there are candidates), then their
  // mask words, first leaves and prefixes.
  auto load_src = [&](i64 c, int32_t* sl) {
#pragma unroll
    for (int k = 0; k < kLivePer; ++k) {
      sl[k] = c < c_end && fm0[k] ? cand_src[c * 27 + (item[k] >> 6)] : -1;
      if (sl[k] >= n_src_lower) {
        set_flag(flags, kFlagInternal);
        sl[k] = -1;
      }
    }
  };
  auto load_words = [&](const int32_t* sl, u64* wd, int32_t* base) {
    int32_t lfirst[kLivePer];
    uint16_t lpre[kLivePer];
#pragma unroll
    for (int k = 0; k < kLivePer; ++k) {
      const i64 ls = sl[k] >= 0 ? sl[k] : 0;
      wd[k] = src_lower_mask[ls * 64 + (item[k] & 63)];
      lfirst[k] = src_lower_first[ls];
      lpre[k] = src_lower_prefix[ls * 64 + (item[k] & 63)];
    }
#pragma unroll
    for (int k = 0; k < kLivePer; ++k) {
      if (sl[k] < 0) wd[k] = 0;
      base[k] = sl[k] >= 0 ? lfirst[k] + lpre[k] : 0;
    }
  };
  i64 c = ncand * xr / 8 + (blockIdx.x >> 3);
  int32_t sl[kLivePer];
  u64 wd[kLivePer];
  int32_t base[kLivePer];
  load_src(c, sl);
  load_words(sl, wd, base);
  for (; c < c_end; c += bpx) {
    int32_t sln[kLivePer];
    load_src(c + bpx, sln);  // next candidate, first level
#pragma unroll
    for (int k = 0; k < kLivePer; ++k)
      if ((item[k] >> 6) == 13 && tid * kLivePer + k < nlive) s_center[item[k] & 63] = wd[k];
    // The co-located source lower (slot 13, every word live) marks its own
    // leaf positions (the box holds offset 0 and a source leaf is never
    // empty): its mask goes into the candidate's as is. A leaf of it whose box
    // neighbours inside the candidate are all source leaves spills only onto
    // positions already marked (or outside the candidate, which are other
    // candidates' to mark), so the leaves of its eroded mask are not visited.
    __syncthreads();
    if (tid < 64) {  // wave 0
      const u64 m = s_center[tid];
      s_mask[tid] = m;
      s_skip[tid] = erode_lower_mask<lo, hi>(m);
    }
    __syncthreads();
    u64 fm[kLivePer];
    int cnt[kLivePer];
    int sum = 0;
#pragma unroll
    for (int k = 0; k < kLivePer; ++k) {
      fm[k] = fm0[k];
      if ((item[k] >> 6) == 13) fm[k] &= ~s_skip[item[k] & 63];
      cnt[k] = popc64(wd[k] & fm[k]);
      sum += cnt[k];
    }
    int total;
    int ex = block_excl_scan<int, 256>(sum, s_wave, total);
#pragma unroll
    for (int k = 0; k < kLivePer; ++k) {
      const int li = tid * kLivePer + k;
      if (li < nlive) {
        s_word[li] = wd[k];
        s_base[li] = base[k];
        s_excl[li] = ex;
        s_item[li] = (uint16_t)item[k];
        s_fm[li] = fm[k];
        for (int j = ex, e = min(ex + cnt[k], kMarkMap); j < e; ++j) s_map[j] = (uint16_t)li;
      }
      ex += cnt[k];
    }
    if (tid == 0) s_excl[nlive] = total;
    __syncthreads();
    // the next candidate's second level, in flight during this one's leaves
    load_words(sln, wd, base);
    for (int k0 = 0; k0 < total; k0 += kMarkIlp * 256) {
      int32_t lf[kMarkIlp];
      uint32_t ps[kMarkIlp];
#pragma unroll
      for (int u = 0; u < kMarkIlp; ++u) {
        const int k = k0 + u * 256 + tid;
        lf[u] = -1;
        ps[u] = 0;
        if (k < total) {
          int a;  // the live item holding reaching leaf k: largest with s_excl[item] <= k
          if (k < kMarkMap) {
            a = s_map[k];
          } else {
            int z = nlive;
            a = 0;
            while (z - a > 1) {
              const int mid = (a + z) >> 1;
              if (s_excl[mid] <= k) a = mid;
              else z = mid;
            }
          }
          const int js = s_item[a] >> 6, w = s_item[a] & 63;
          const u64 word = s_word[a];
          const int bit = select_bit(word & s_fm[a], k - s_excl[a]);
          const i64 leaf = (i64)s_base[a] + popc64(word & ((1ull << bit) - 1));
          if (leaf < 0 || leaf >= n_src_leaf) {
            set_flag(flags, kFlagInternal);
          } else {
            lf[u] = (int32_t)leaf;
            ps[u] = pack_pos((w >> 2) + 16 * (js / 9 - 1), (w & 3) * 4 + (bit >> 4) + 16 * ((js / 3) % 3 - 1),
                             (bit & 15) + 16 * (js % 3 - 1));
          }
        }
      }
      u64 W[kMarkIlp][8];  // leaf 0 stands in for an empty item (its marks are skipped)
#pragma unroll
      for (int u = 0; u < kMarkIlp; ++u)
#pragma unroll
        for (int q = 0; q < 8; ++q) W[u][q] = src_leaf_mask[(i64)(lf[u] >= 0 ? lf[u] : 0) * 8 + q];
#pragma unroll
      for (int u = 0; u < kMarkIlp; ++u)
        if (lf[u] >= 0) mark_box_leaf(W[u], ps[u], lo, hi, s_mask);
    }
    __syncthreads();
    if (tid < 64) store_candidate(c, s_mask[tid], cand_child, cand_prefix, cand_counts);  // wave 0
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kLivePer; ++k) sl[k] = sln[k];
  }
}

// Workgroups of k_leaf_mark_box<lo, hi> resident at once on the current device:
// its CUs times the kernel's workgroups per CU (read once per instantiation).
template <int lo, int hi>
static i64 mark_box_resident() {
  static std::atomic<int> per_cu{0};
  int n = per_cu.load(std::memory_order_relaxed);
  if (n <= 0) {
    hip_check(hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_leaf_mark_box<lo, hi>, 256, 0),
              "hipOccupancyMaxActiveBlocksPerMultiprocessor");
    n = n > 0 ? n : 1;
    per_cu.store(n, std::memory_order_relaxed);
  }
  return (i64)device_cu_count() * n;
}

// ------------------------------------------------------------------ writers: leaf masks (pass B)
// Index of the source leaf at position p inside source lower s, or -1 when that
// leaf is absent (or s / the result is out of range, which also flags an error).
__device__ __forceinline__ int32_t src_leaf(const u64* lower_mask, const uint16_t* lower_prefix,
                                            const int32_t* lower_first, int32_t s, i64 px, i64 py, i64 pz,
                                            int32_t n_lower, int32_t n_leaf, int32_t* flags) {
  if (s < 0 || s >= n_lower) {
    set_flag(flags, kFlagInternal);
    return -1;
  }
  const int bit = (int)((px * 16 + py) * 16 + pz);
  const int w = bit >> 6, b = bit & 63;
  const u64 word = lower_mask[(i64)s * 64 + w];
  if (!((word >> b) & 1ull)) return -1;
  const int32_t r = lower_first[s] + lower_prefix[(i64)s * 64 + w] + popc64(word & ((1ull << b) - 1));
  if (r < 0 || r >= n_leaf) {
    set_flag(flags, kFlagInternal);
    return -1;
  }
  return r;
}

// Nibble (4 bits) -> byte with every bit doubled.
__device__ __forceinline__ u64 double_bits4(u64 b) {
  b = (b | (b << 2)) & 0x33ull;
  b = (b | (b << 1)) & 0x55ull;
  return b | (b << 1);
}

// Refine: output rows 2r, 2r+1 and bits 2c, 2c+1 come from row 4qy + r, bit 4qz + c of w.
// The four source rows are the 32-bit half qy of w (one byte each); their nibble
// qz, one per byte, has every bit doubled in place, and each byte then fills two
// 8-bit output rows.
__device__ __forceinline__ u64 refine_word(u64 w, int qy, int qz) {
  uint32_t t = (uint32_t)(w >> (32 * qy));
  t = (t >> (4 * qz)) & 0x0f0f0f0fu;   // nibble of row r in byte r
  t = (t | (t << 2)) & 0x33333333u;    // bits 0..3 -> 0, 1, 4, 5
  t = (t | (t << 1)) & 0x55555555u;    // -> 0, 2, 4, 6
  t |= t << 1;                         // doubled: byte r = row 2r's bits
  const uint32_t lo = (t & 0xffu) | ((t & 0xff00u) << 8);            // rows 0, 1 -> bytes 0, 2
  const uint32_t hi = ((t >> 16) & 0xffu) | ((t >> 8) & 0xff0000u);  // rows 2, 3 -> bytes 0, 2
  return ((u64)(hi | (hi << 8)) << 32) | (lo | (lo << 8));           // each byte twice
}

// Coarsen: OR each 2x2x2 block of the source into one bit, giving a 4^3 block
// placed at offset 4q of the output leaf.
__device__ __forceinline__ void coarsen_place(u64 out[8], const u64 W[8], const I3& q) {
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    u64 v = W[2 * x] | W[2 * x + 1];
    v = (v | (v >> 1)) & 0x5555555555555555ull;  // z pairs -> even bits
    v = (v | (v >> 8)) & 0x00ff00ff00ff00ffull;  // y pairs -> even bytes
    v = (v | (v >> 1)) & 0x3333333333333333ull;  // even bits 0,2,4,6 -> 0,1,4,5
    v = (v | (v >> 2)) & 0x0f0f0f0f0f0f0f0full;  // -> 0..3
    u64 placed = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) placed |= ((v >> (16 * r)) & 0xfull) << ((4 * q.y + r) * 8 + 4 * q.z);
    // constant indices keep `out` in registers (a runtime index would put it in scratch memory)
    out[x] |= q.x ? 0ull : placed;
    out[4 + x] |= q.x ? placed : 0ull;
  }
}

// Output leaf masks by gathering from the source leaves that feed them: the
// unique parent (refine) or the 8 children (coarsen; box ops have their own
// separable gather below). Coarsen splits the sources of one output leaf over 4
// adjacent lanes and ORs the partial masks with shuffles, so the dependent
// lookups run in parallel. Also writes the leaf's prefix word, packed local bbox
// and in-run voxel count.
// KIND: 0 refine, 1 coarsen; one instantiation each.
// Output leaf count on the device (the counts stage's total; a launch may be
// sized by a capacity above it): clamped to the capacity, with a flag if above.
__device__ __forceinline__ i64 device_count(const int32_t* d_n, i64 cap, int32_t* flags) {
  i64 n = *d_n;
  if (n < 0 || n > cap) {
    if (blockIdx.x == 0 && threadIdx.x == 0) set_flag(flags, kFlagInternal);
    n = n < 0 ? 0 : cap;
  }
  return n;
}

template <int KIND>
__global__ void __launch_bounds__(256) k_leaf_gather(const int4* out_origin, const int32_t* leaf_cand,
                                                     const int32_t* d_n, i64 n_cap, const int32_t* cand_src,
                                                     const u64* src_lower_mask, const uint16_t* src_lower_prefix,
                                                     const int32_t* src_lower_first, const u64* src_leaf_mask,
                                                     int32_t n_src_lower, int32_t n_src_leaf,
                                                     const int32_t* d_num_cands, u64* out_mask, u64* out_prefix,
                                                     uint32_t* leaf_box, int32_t* leaf_inrun,
                                                     i64* vox_part, int32_t* flags) {
  constexpr int lpl = KIND == 0 ? 1 : 4;  // lanes per output leaf
  const i64 n = device_count(d_n, n_cap, flags);
  if ((i64)blockIdx.x * (256 / lpl) >= n) return;  // past the leaves (uniform per block)
  const i64 lblk = blockIdx.x;
  const i64 gt = lblk * 256 + threadIdx.x;
  const i64 i = gt / lpl;
  const int sub = (int)(gt % lpl);
  bool valid = i < n;
  u64 out[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) out[k] = 0;
  i64 c = -1;
  int4 o = make_int4(0, 0, 0, 0);
  if (valid) {
    o = out_origin[i];
    c = leaf_cand[i];
    if (c < 0 || c >= *d_num_cands) {
      set_flag(flags, kFlagInternal);
      valid = false;
    }
  }
  if (valid) {
    const i64 ax = o.x >> 3, ay = o.y >> 3, az = o.z >> 3;  // output leaf coordinates
    const i64 lx = ax & 15, ly = ay & 15, lz = az & 15;
    if constexpr (KIND == 0) {
      const int32_t s = cand_src[c];
      const int32_t src = src_leaf(src_lower_mask, src_lower_prefix, src_lower_first, s, (ax >> 1) & 15,
                                   (ay >> 1) & 15, (az >> 1) & 15, n_src_lower, n_src_leaf, flags);
      if (src < 0) {
        set_flag(flags, kFlagInternal);
      } else {
        u64 W[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) W[k] = src_leaf_mask[(i64)src * 8 + k];
        const int qx = (int)(ax & 1), qy = (int)(ay & 1), qz = (int)(az & 1);
#pragma unroll
        for (int x = 0; x < 8; ++x) out[x] = refine_word(W[4 * qx + (x >> 1)], qy, qz);
      }
    } else if constexpr (KIND == 1) {
      const int32_t s = cand_src[c * 8 + octant_index(lx >> 3, ly >> 3, lz >> 3)];
      if (s < 0) set_flag(flags, kFlagInternal);
      for (int j = sub; j < 8 && s >= 0; j += 4) {
        const I3 q = octant(j);
        const int32_t src = src_leaf(src_lower_mask, src_lower_prefix, src_lower_first, s, (2 * lx + q.x) & 15,
                                     (2 * ly + q.y) & 15, (2 * lz + q.z) & 15, n_src_lower, n_src_leaf, flags);
        if (src < 0) continue;
        u64 W[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) W[k] = src_leaf_mask[(i64)src * 8 + k];
        coarsen_place(out, W, q);
      }
    }
  }
  if constexpr (lpl == 4) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      out[k] |= __shfl_xor(out[k], 1, kWave);
      out[k] |= __shfl_xor(out[k], 2, kWave);
    }
  }
  const bool writer = i < n && sub == 0;
  u64 prefix = 0;
  int count = 0;
  uint32_t box = kEmptyBox;
  if (writer && valid) {
#pragma unroll
    for (int k = 0; k < 8; ++k) out_mask[i * 8 + k] = out[k];
    leaf_stats(out, prefix, count, box);
    out_prefix[i] = prefix;
  }
  // voxels before this leaf within the block's leaves, and the block's total
  const int32_t inrun = block_run_scan(count, &vox_part[lblk]);
  if (writer) {
    leaf_box[i] = box;
    leaf_inrun[i] = inrun;
  }
}

// ------------------------------------------------------------------ writers: box ops, separable
// A box [lo, hi]^3 is the Minkowski sum of three axis segments, so an output
// leaf's mask is the source set dilated along x, then y, then z, restricted to
// the leaf. The x pass runs on each needed source column (y, z leaf offset), the
// y pass on each needed z offset, the z pass once; each pass shifts whole 64-bit
// words, and a neighbour leaf only ever supplies its boundary word / row / bit.
// Four lanes share an output leaf, lane k owning output words 2k and 2k+1: the
// y and z passes never mix words, and the x pass needs just one more word on
// each side (from the x-neighbour leaf at the ends). The source lookups are
// split over the four lanes and their results exchanged with shuffles.
// Raw buffer loads (the kBuf form, for source arrays under 2 GiB): 32-bit byte
// offsets off one resource, and an offset past the array (kOff) reads zeros, so
// a missing source costs no select. The resource's third word is the gfx9
// family's raw-buffer format word.
constexpr uint32_t kOff = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}

// kBuf: the source arrays and the candidate table are read through buffer
// resources (each under 2 GiB, checked by the host); otherwise through 64-bit
// addresses, with index 0 standing in for a missing source and a select after.
template <int lo, int hi, bool kBuf>  // the box [lo, hi]^3: dilate [-1, 1], pads [-1, 0] and [0, 1]
__global__ void __launch_bounds__(256) k_leaf_gather_box(const int4* out_origin, const int32_t* leaf_cand,
                                                         const int32_t* d_n, i64 n_cap, const int32_t* cand_src,
                                                         const u64* src_lower_mask, const uint16_t* src_lower_prefix,
                                                         const int32_t* src_lower_first, const u64* src_leaf_mask,
                                                         int32_t n_src_lower, int32_t n_src_leaf,
                                                         const int32_t* d_num_cands, u64* out_mask, u64* out_prefix,
                                                         uint32_t* leaf_box, int32_t* leaf_inrun,
                                                         i64* vox_part, int32_t* flags, uint32_t cand_src_bytes) {
  const i64 n = device_count(d_n, n_cap, flags);
  const i64 nb = (n * 4 + 255) / 256;  // workgroups that hold leaves (the launch may hold more)
  if ((i64)blockIdx.x >= nb) return;  // uniform per block
  const i64 lblk = xcd_block(blockIdx.x, nb);  // contiguous leaves per XCD (shared source leaves)
  const i64 gt = lblk * 256 + threadIdx.x;
  const i64 i = gt >> 2;
  const int sub = (int)(gt & 3);
  [[maybe_unused]] __amdgpu_buffer_rsrc_t r_cand, r_lmask, r_lpre, r_lfirst, r_leaf;
  if constexpr (kBuf) {
    r_cand = buf_rsrc(cand_src, cand_src_bytes);
    r_lmask = buf_rsrc(src_lower_mask, (uint32_t)n_src_lower * 512u);
    r_lpre = buf_rsrc(src_lower_prefix, (uint32_t)n_src_lower * 128u);
    r_lfirst = buf_rsrc(src_lower_first, (uint32_t)n_src_lower * 4u);
    r_leaf = buf_rsrc(src_leaf_mask, (uint32_t)n_src_leaf * 64u);
  }
  // Every load goes to a valid index (n, the candidates, the source lowers and
  // leaves are all non-empty here; index 0 stands in for a missing one, or an
  // offset past a buffer) and is masked afterwards, so each level's loads are in
  // flight together. Indices fit 32 bits (source lowers < 2^25, checked by the host).
  const int32_t ncand = *d_num_cands;
  const int32_t ic = (int32_t)(i < n ? i : n - 1);
  const int4 o = out_origin[ic];
  int32_t c = leaf_cand[ic];
  bool valid = i < n;
  bool bad = valid && (c < 0 || c >= ncand);
  valid = valid && !bad;
  if (!valid) c = 0;
  const int lx = (o.x >> 3) & 15, ly = (o.y >> 3) & 15, lz = (o.z >> 3) & 15;
  // The source leaves of this output leaf sit at leaf offsets s in [-hi, -lo]^3
  // (W^3 of them), numbered k = ((sx+hi)*W + (sy+hi))*W + (sz+hi); lane `sub`
  // resolves k = sub + 4q, level by level so that the loads overlap. The
  // offsets of slot q for the four lanes come from one packed constant.
  constexpr int W = hi - lo + 1, NK = W * W * W, kPer = (NK + 3) / 4;
  int32_t sl[kPer], bit[kPer];
  bool use[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    uint32_t pack = 0;  // per lane: (sx+hi) | (sy+hi) << 2 | (sz+hi) << 4 | used << 6
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      const int k = 4 * q + l;
      if (k < NK) pack |= (uint32_t)((k / (W * W)) | (((k / W) % W) << 2) | ((k % W) << 4) | 64) << (8 * l);
    }
    const uint32_t code = (pack >> (8 * sub)) & 0xffu;
    use[q] = valid && (code & 64u);
    const int px = lx + (int)(code & 3u) - hi, py = ly + (int)((code >> 2) & 3u) - hi, pz = lz + (int)((code >> 4) & 3u) - hi;
    bit[q] = ((px & 15) * 16 + (py & 15)) * 16 + (pz & 15);
    const int slot = index27(px >> 4, py >> 4, pz >> 4);
    if constexpr (kBuf) {
      sl[q] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(r_cand, use[q] ? (uint32_t)(c * 27 + slot) * 4u : kOff, 0, 0);
    } else {
      sl[q] = cand_src[c * 27 + (use[q] ? slot : 13)];
    }
  }
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    bad |= use[q] && sl[q] >= n_src_lower;
    if (!use[q] || sl[q] >= n_src_lower) sl[q] = -1;
  }
  u64 word[kPer];
  int32_t lfirst[kPer];
  uint16_t lpre[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const uint32_t w = (uint32_t)(bit[q] >> 6);
    if constexpr (kBuf) {  // a missing source reads zeros
      const uint32_t at = sl[q] >= 0 ? (uint32_t)sl[q] * 64u + w : kOff / 8u;
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(r_lmask, at * 8u, 0, 0);
      word[q] = ((u64)v[1] << 32) | v[0];
      lfirst[q] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(r_lfirst, sl[q] >= 0 ? (uint32_t)sl[q] * 4u : kOff, 0, 0);
      lpre[q] = __builtin_amdgcn_raw_buffer_load_b16(r_lpre, at * 2u, 0, 0);
    } else {
      const uint32_t ls = sl[q] >= 0 ? (uint32_t)sl[q] : 0u;
      word[q] = src_lower_mask[ls * 64u + w];
      lfirst[q] = src_lower_first[ls];
      lpre[q] = src_lower_prefix[ls * 64u + w];
      if (sl[q] < 0) word[q] = 0;
    }
  }
  int32_t r[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int b = bit[q] & 63;
    const bool hit = (word[q] >> b) & 1ull;  // zero word for a missing source
    r[q] = lfirst[q] + lpre[q] + popc64(word[q] & ((1ull << b) - 1));
    const bool out_of_range = hit && (uint32_t)r[q] >= (uint32_t)n_src_leaf;
    bad |= out_of_range;
    if (!hit || out_of_range) r[q] = -1;
  }
  if (bad) set_flag(flags, kFlagInternal);
  // Source rows: lane `sub` loads words 2sub and 2sub+1 of every needed row
  // (sy, sz) of the centre column of source leaves (one 16-byte load), lane 0
  // also word 7 of the row's x-1 leaf and lane 3 word 0 of its x+1 leaf; the
  // words 2sub-1 and 2sub+2 come from the neighbouring lanes of the quad.
  // Leaf indices resolved by other lanes of the quad arrive by quad broadcasts.
  // Every row's leaf indices come first (quad broadcasts), then the loads of
  // one z offset's rows are issued together, before any of their quad
  // permutations (the compiler moves no load across those).
  int32_t rcs[3][3], res[3][3];  // [sz + 1][sy + 1]: centre and edge leaf of the row
#pragma unroll
  for (int sz = -1; sz <= 1; ++sz)
#pragma unroll
    for (int sy = -1; sy <= 1; ++sy) {
      rcs[sz + 1][sy + 1] = -1;
      res[sz + 1][sy + 1] = -1;
      if (sz < -hi || sz > -lo || sy < -hi || sy > -lo) continue;
      // source leaves at (sx, sy, sz), sx = -1, 0, 1 (the ones in the box): slot k
      constexpr int kNone = -1;
      const int ky = sy + hi, kz = sz + hi;
      const int kc = ((0 + hi) * W + ky) * W + kz;   // sx = 0
      const int km = ((-1 + hi) * W + ky) * W + kz;  // sx = -1 (hi > 0)
      const int kp = ((1 + hi) * W + ky) * W + kz;   // sx = +1 (lo < 0)
      rcs[sz + 1][sy + 1] = quad_bcast32(r[kc >> 2], kc & 3);
      const int32_t rm = hi > 0 ? quad_bcast32(r[km >> 2], km & 3) : kNone;
      const int32_t rp = lo < 0 ? quad_bcast32(r[kp >> 2], kp & 3) : kNone;
      res[sz + 1][sy + 1] = sub == 0 ? rm : (sub == 3 ? rp : kNone);  // edge leaf of this lane
    }
  u64 ys[3][2];
#pragma unroll
  for (int sz = -1; sz <= 1; ++sz) {
    u64 xs[3][2] = {{0, 0}, {0, 0}, {0, 0}};
    u64 wa[3] = {0, 0, 0}, wb[3] = {0, 0, 0}, we[3] = {0, 0, 0};
#pragma unroll
    for (int sy = -1; sy <= 1; ++sy) {
      if (sz < -hi || sz > -lo || sy < -hi || sy > -lo) continue;
      const int32_t rc = rcs[sz + 1][sy + 1], re = res[sz + 1][sy + 1];
      if constexpr (kBuf) {  // a missing leaf reads zeros
        const auto own = __builtin_amdgcn_raw_buffer_load_b128(r_leaf, rc >= 0 ? (uint32_t)rc * 64u + (uint32_t)sub * 16u : kOff, 0, 0);
        const auto edge = __builtin_amdgcn_raw_buffer_load_b64(r_leaf, re >= 0 ? (uint32_t)re * 64u + (sub == 0 ? 56u : 0u) : kOff, 0, 0);
        wa[sy + 1] = ((u64)own[1] << 32) | own[0];
        wb[sy + 1] = ((u64)own[3] << 32) | own[2];
        we[sy + 1] = ((u64)edge[1] << 32) | edge[0];
      } else {
        const ulonglong2 own = reinterpret_cast<const ulonglong2*>(src_leaf_mask)[(i64)(rc >= 0 ? rc : 0) * 4 + sub];
        const u64 edge = src_leaf_mask[(i64)(re >= 0 ? re : 0) * 8 + (sub == 0 ? 7 : 0)];
        wa[sy + 1] = rc >= 0 ? (u64)own.x : 0ull;
        wb[sy + 1] = rc >= 0 ? (u64)own.y : 0ull;
        we[sy + 1] = re >= 0 ? edge : 0ull;
      }
    }
#pragma unroll
    for (int sy = -1; sy <= 1; ++sy) {
      if (sz < -hi || sz > -lo || sy < -hi || sy > -lo) continue;
      // The permutations run on the whole quad before the selects (a select
      // around them would make them conditional, and lane 0 or 3 then absent).
      const u64 pl = quad_perm64<0, 0, 1, 2>(wb[sy + 1]), pr = quad_perm64<1, 2, 3, 3>(wa[sy + 1]);
      const u64 left = sub == 0 ? we[sy + 1] : pl;   // word 2sub - 1
      const u64 right = sub == 3 ? we[sy + 1] : pr;  // word 2sub + 2
      xs[sy + 1][0] = wa[sy + 1] | (hi > 0 ? left : 0ull) | (lo < 0 ? wb[sy + 1] : 0ull);
      xs[sy + 1][1] = wb[sy + 1] | (hi > 0 ? wa[sy + 1] : 0ull) | (lo < 0 ? right : 0ull);
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      u64 v = xs[1][e];
      if (hi > 0) v |= (xs[1][e] << 8) | (xs[0][e] >> 56);
      if (lo < 0) v |= (xs[1][e] >> 8) | (xs[2][e] << 56);
      ys[sz + 1][e] = v;
    }
  }
  u64 outw[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    u64 v = ys[1][e];
    if (hi > 0) v |= ((ys[1][e] & ~kZ7) << 1) | ((ys[0][e] & kZ7) >> 7);
    if (lo < 0) v |= ((ys[1][e] & ~kZ0) >> 1) | ((ys[2][e] & kZ0) << 7);
    outw[e] = valid ? v : 0ull;
  }
  // leaf statistics from the quad's 8 words (lane s: words 2s, 2s+1)
  u64 prefix;
  int count;
  uint32_t box;
  quad_leaf_stats(outw[0], outw[1], sub, prefix, count, box);
  if (i < n && valid) {
    reinterpret_cast<ulonglong2*>(out_mask)[i * 4 + sub] = make_ulonglong2(outw[0], outw[1]);
    if (sub == 0) out_prefix[i] = prefix;
  }
  // voxels before this leaf within the block's leaves, and the block's total
  const int32_t inrun = block_run_scan(sub == 0 && i < n ? count : 0, &vox_part[lblk]);
  if (i < n && sub == 0) {
    leaf_box[i] = box;
    leaf_inrun[i] = inrun;
  }
}

// ------------------------------------------------------------------ masked refine
// Keep flags (one byte per voxel, in enumeration order) -> masked copies of the
// source leaf masks. One wave per leaf: lane r owns row r = x*8 + y (byte y of
// word x); a wave scan of the row popcounts gives each row's first voxel, the
// lane keeps the bits whose flags are set, and the 8 lanes of a word OR their
// rows together.
__global__ void __launch_bounds__(256) k_mask_leaves(const tc_grid_header* hdr, const int4* leaf_origin,
                                                     const u64* leaf_mask, const i64* leaf_offset,
                                                     const uint8_t* keep, i64 n_keep, i64 n_leaf, u64* out_mask,
                                                     int32_t B, int32_t* flags) {
  const i64 l = (i64)blockIdx.x * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (l >= n_leaf) return;  // uniform per wave; no block barrier
  const int x = lane >> 3, y = lane & 7;
  const uint32_t row = (uint32_t)(leaf_mask[l * 8 + x] >> (8 * y)) & 0xffu;
  const int cnt = __popc(row);
  const int before = wave_incl_scan(cnt) - cnt;
  const int g = leaf_origin[l].w;
  i64 base = -1;
  if (g >= 0 && g < B) base = hdr[g].voxel_begin + leaf_offset[l] + before;
  uint32_t kept = 0;
  int k = 0;
  for (uint32_t m = row; m; m &= m - 1, ++k) {
    const i64 j = base + k;
    if (base < 0 || j >= n_keep) {
      set_flag(flags, kFlagInternal);
      break;
    }
    if (keep[j]) kept |= m & (~m + 1);  // lowest set bit of m
  }
  u64 w = (u64)kept << (8 * y);
  w |= __shfl_xor(w, 1, kWave);
  w |= __shfl_xor(w, 2, kWave);
  w |= __shfl_xor(w, 4, kWave);
  if (y == 0) out_mask[l * 8 + x] = w;
}

void mask_leaves(const tc_grid_batch* src, const uint8_t* keep, i64 n_keep, u64* out_mask, int32_t* flags,
                 hipStream_t s) {
  const GridView v = src->view();
  launch("k_mask_leaves", k_mask_leaves, ceil_div((i64)v.n_leaf, 4), 256, s, (const tc_grid_header*)v.headers,
         (const int4*)v.leaf_origin, (const u64*)v.leaf_mask, (const i64*)v.leaf_offset, keep, n_keep,
         (i64)v.n_leaf, out_mask, v.B, flags);
}

// ------------------------------------------------------------------ driver
// Output layouts by capacity are taken while they stay under this size.
constexpr size_t kBoundedBytes = size_t(32) << 20;

static void check_pass_flags(int32_t f) {
  if (f & kFlagSource)
    throw Error(TC_ERR_INTERNAL, "the source batch failed a device consistency check when it was written");
  if (f & kFlagOverflow) throw Error(TC_ERR_OVERFLOW, "an output voxel coordinate leaves int32");
  if (f & kFlagInternal) throw Error(TC_ERR_INTERNAL, "pass: device consistency check failed");
}

void resolve_counts(const tc_grid_batch* cb) {
  if (!cb->hdr_pending) return;
  tc_grid_batch* b = const_cast<tc_grid_batch*>(cb);
  auto release = [&]() {
    pinned_block_give(b->hdr_host, b->hdr_host_cap);
    pending_event_give(b->device, b->hdr_ev);
    b->hdr_host = nullptr;
    b->hdr_host_cap = 0;
    b->hdr_ev = nullptr;
    b->hdr_pending = false;
  };
  try {
    hip_check(hipEventSynchronize(b->hdr_ev), "hipEventSynchronize");
    const char* h = static_cast<const char*>(b->hdr_host);
    check_pass_flags(*reinterpret_cast<const int32_t*>(h + sizeof(tc_grid_header) * (size_t)b->B));
    set_counts_from_headers(b, reinterpret_cast<const tc_grid_header*>(h));
  } catch (...) {
    release();
    throw;
  }
  release();
}

tc_grid_batch* build_pass(const tc_grid_batch* src, int op, const OutAlloc& oa, const u64* leaf_mask_override,
                          bool defer) {
  resolve_counts(src);  // a source whose headers are still on their way
  const OpInfo oi = op_info(op);
  hipStream_t s = oa.stream;
  const int32_t B = src->B;
  GridView sv = src->view();
  if (leaf_mask_override) sv.leaf_mask = const_cast<u64*>(leaf_mask_override);
  const i64 nT = (i64)src->n2 * oi.m;
  const i64 nL = (i64)src->n1 * oi.m;
  if (nT > 0x7fffffffLL || nL > 0x7fffffffLL || nL * oi.m_src > (1ll << 40) || src->n1 >= (1 << 25))
    throw Error(TC_ERR_UNSUPPORTED, "pass: source batch too large");

  const bool small_tiles = nT > 0 && nT <= kTilesMax;
  const bool small_lowers = small_tiles && nT <= kLowersSmallTiles && nL > 0 && nL <= kLowersSmallMax &&
                            (op == TC_OP_COARSEN || nL / oi.m <= kReachMax);
  // Small batches (a tile stage in one workgroup; the lower stage in one
  // workgroup too, or in its multi-launch form) lay the output out by
  // capacities known before any launch (a
  // source leaf feeds at most 8 / 1 / 27 / 8 output leaves for refine, coarsen,
  // dilate, pads; the tile and lower candidates bound the nodes), so the output
  // is allocated while the node, marking and count stages run (they do not touch
  // it) and the writers follow the counts stage without a host round trip; the
  // one readback (headers and status) ends the pass.
  const i64 per_leaf = op == TC_OP_REFINE ? 8 : (op == TC_OP_COARSEN ? 1 : oi.m);
  const i64 gran = op == TC_OP_REFINE ? 256 : 64;  // leaves per gather workgroup (voxel-sum runs)
  const i64 L_cap = (i64)src->nl * per_leaf;
  const bool bounded = small_tiles && nL > 0 && L_cap > 0 && L_cap <= 0x7fffffffLL &&
                       finalize_small_fits(L_cap, B, gran) && make_layout(B, nT, nL, L_cap).total <= kBoundedBytes;
  tc_grid_batch* out = nullptr;
  try {
    Arena a(s);
    const i64 nTs = small_tiles ? 0 : nT;  // sort scratch only for the multi-kernel tile path
    const size_t o_keys = a.reserve(sizeof(Key128) * nTs);
    const size_t o_vals = a.reserve(4 * nTs);
    const size_t o_head = a.reserve(4 * nTs);
    const size_t o_texcl = a.reserve(4 * (nTs + 1));
    const size_t o_toc = a.reserve(4 * nT);
    const size_t o_ntiles = a.reserve(4);
    const size_t o_ncand = a.reserve(4);
    const size_t o_utile = a.reserve(16 * nT);
    const size_t o_tchild = a.reserve(4096 * nT);
    const size_t o_tpre = a.reserve(1024 * nT);
    const size_t o_tlc = a.reserve(4 * nT);
    const size_t o_tlb = a.reserve(4 * (nT + 1));
    const size_t o_tne = a.reserve(4 * nT);
    const size_t o_uex = a.reserve(4 * (nT + 1));
    const size_t o_gtb = a.reserve(4 * ((i64)B + 1));
    const size_t o_corig = a.reserve(16 * nL);
    const size_t o_cchild = a.reserve(512 * nL);
    const size_t o_cpre = a.reserve(128 * nL);
    const size_t o_ccnt = a.reserve(8 * nL);
    const size_t o_cscan = a.reserve(8 * (nL + 1));
    const size_t o_nbr = a.reserve(4 * nL);
    const size_t o_csrc = a.reserve(4 * nL * oi.m_src);
    const size_t o_ginfo = a.reserve(4 * 6 * (i64)B);
    const size_t o_rb = a.reserve(4 * (5 + 3 * (i64)B));  // readback words, then the rank stage's counter
    const size_t o_ureach = a.reserve(4 * (i64)src->n2);
    const size_t o_lreach = a.reserve(4 * (i64)src->n1);
    const size_t o_stmp = a.reserve(std::max(scan_tmp_bytes(nT, 4), scan_tmp_bytes(nL, 8)));
    a.commit();

    TreeScratch ts{};
    ts.cap_tiles = nT;
    ts.cap_cands = nL;
    ts.d_num_tiles = a.at<int32_t>(o_ntiles);
    ts.utile = a.at<int4>(o_utile);
    ts.tile_child = a.at<u64>(o_tchild);
    ts.tile_prefix = a.at<uint16_t>(o_tpre);
    ts.tile_lower_count = a.at<int32_t>(o_tlc);
    ts.tile_lower_base = a.at<int32_t>(o_tlb);
    ts.tile_nonempty = a.at<int32_t>(o_tne);
    ts.upper_excl = a.at<int32_t>(o_uex);
    ts.grid_tile_begin = a.at<int32_t>(o_gtb);
    ts.d_num_cands = a.at<int32_t>(o_ncand);
    ts.cand_origin = a.at<int4>(o_corig);
    ts.cand_child = a.at<u64>(o_cchild);
    ts.cand_prefix = a.at<uint16_t>(o_cpre);
    ts.cand_counts = a.at<i64>(o_ccnt);
    ts.cand_scan = a.at<i64>(o_cscan);
    ts.grid_info = a.at<int32_t>(o_ginfo);
    ts.readback = a.at<int32_t>(o_rb);
    ts.scan_tmp = a.at<char>(o_stmp);
    ts.flags = ts.readback;
    int32_t* rank_ctr = ts.readback + 4 + 3 * B;
    int32_t* tile_of_cand = a.at<int32_t>(o_toc);
    int32_t* lower_nbr = a.at<int32_t>(o_nbr);
    int32_t* cand_src = a.at<int32_t>(o_csrc);

    // tiles
    // box ops on small batches: voxel-exact face reach sets of uppers and lowers
    const bool box_op = op != TC_OP_REFINE && op != TC_OP_COARSEN;
    uint32_t* box_lreach = nullptr;
    uint32_t* lreach_early = nullptr;  // lower reach sets computed with the uppers' (one launch)
    if (box_op && small_tiles && src->n1 <= kBoxReachLowers) {
      box_lreach = a.at<uint32_t>(o_lreach);
      launch("k_box_reach", k_box_reach, src->n2, 256, s, (const int32_t*)sv.upper_first, (int32_t)src->n2,
             (const int32_t*)sv.lower_first, (int32_t)src->n1, (const int4*)sv.leaf_origin,
             (const int32_t*)sv.leaf_parent, (const u64*)sv.leaf_mask, (int32_t)src->nl, op, oi.m,
             a.at<uint32_t>(o_ureach), box_lreach);
    }
    if (small_tiles) {
      // the bitmaps are zeroed in-kernel (only the live tiles') by the fused
      // lower stage, or here when few are expected: at most 1 MiB of capacity,
      // or refine's at most 8 tiles per source upper (up to 4 MiB), or box ops
      // with voxel-exact reach (only uppers with voxels on a face reach a
      // neighbour tile; up to 8 MiB of capacity); otherwise by a wide fill
      const bool zero_here = !small_lowers && (nT <= 256 || (op == TC_OP_REFINE && nT <= 1024) ||
                                               (box_lreach != nullptr && nT <= 2048));
      // more source uppers than one round of the tile stage's in-kernel reach (64:
      // sixteen waves of four): their reach sets in a wide launch first
      uint32_t* ureach = box_lreach ? a.at<uint32_t>(o_ureach) : nullptr;
      if (!box_lreach && op != TC_OP_COARSEN && src->n2 > 64) {
        ureach = a.at<uint32_t>(o_ureach);
        // the multi-launch lower stage's reach sets come from the same launch
        const i64 ub = ceil_div((i64)src->n2, 4);
        const i64 nlo = small_lowers ? 0 : (i64)src->n1;
        if (nlo > 0) lreach_early = a.at<uint32_t>(o_lreach);
        launch("k_node_reach", k_node_reach, ub + ceil_div(nlo, 4), 256, s, (const u64*)sv.upper_mask,
               (i64)src->n2, 512, op, oi.m, ureach, ub, (const u64*)sv.lower_mask, nlo, lreach_early);
      }
      if (small_lowers) {  // the lower stage follows in the same workgroup
        launch("k_nodes_small", k_nodes_small, 1, kTilesThreads, s, (const int4*)sv.upper_origin,
               (const u64*)sv.upper_mask, (int32_t)src->n2, B, ts.utile, ts.grid_tile_begin,
               (const uint32_t*)ureach, ts.readback, (const int32_t*)sv.status, (const int4*)sv.lower_origin,
               (const u64*)sv.lower_mask, nL, op, oi.m, oi.m_src, tile_of_cand, ts.d_num_tiles, ts.tile_child,
               ts.tile_prefix, ts.tile_lower_base, ts.d_num_cands, ts.cand_child, lower_nbr, ts.cand_origin, cand_src,
               (const uint32_t*)box_lreach);
      } else {
        launch("k_tiles_small", k_tiles_small, 1, kTilesThreads, s, (const int4*)sv.upper_origin,
               (const u64*)sv.upper_mask, (int32_t)src->n2, op, oi.m, B, ts.utile, tile_of_cand, ts.d_num_tiles,
               ts.grid_tile_begin, ts.tile_child, zero_here ? 1 : 0, (const uint32_t*)ureach, ts.readback,
               (const int32_t*)sv.status, rank_ctr);
        if (!zero_here) fill_u64(ts.tile_child, 0, nT * 512, ts.d_num_tiles, 512, s);
      }
    } else {
      launch("k_flags_from_source", k_flags_from_source, 1, 64, s, ts.readback, (const int32_t*)sv.status);
      if (nT > 0) {
        Key128* keys = a.at<Key128>(o_keys);
        uint32_t* vals = a.at<uint32_t>(o_vals);
        int32_t* head = a.at<int32_t>(o_head);
        int32_t* texcl = a.at<int32_t>(o_texcl);
        launch("k_tile_candidates", k_tile_candidates, ceil_div(nT, 256), 256, s, (const int4*)sv.upper_origin, nT,
               op, oi.m, keys, vals);
        sort_pairs_128(keys, vals, nT, tile_key_bits(B), s);
        launch("k_tile_heads", k_tile_heads, ceil_div(nT, 256), 256, s, (const Key128*)keys, nT, head);
        scan_excl_i32(head, texcl, nT, nullptr, s, ts.d_num_tiles, ts.scan_tmp);
        launch("k_tile_scatter", k_tile_scatter, ceil_div(nT, 256), 256, s, (const Key128*)keys,
               (const uint32_t*)vals, (const int32_t*)head, (const int32_t*)texcl, nT, ts.utile, tile_of_cand,
               ts.flags);
      } else {
        fill_i32(ts.d_num_tiles, 0, 1, nullptr, 1, s);
      }
      tree_tile_ranges(ts, B, s);
      fill_u64(ts.tile_child, 0, nT * 512, ts.d_num_tiles, 512, s);
    }
    // lowers. The candidate -> source table starts empty; refine and the box ops
    // store every word of their candidates' leaf masks, coarsen ORs into zeros.
    if (!small_lowers) {
      uint32_t* lreach = box_lreach ? box_lreach : lreach_early;
      if (!lreach && op != TC_OP_COARSEN) {
        lreach = a.at<uint32_t>(o_lreach);
        const i64 lb = ceil_div((i64)src->n1, 4);
        launch("k_node_reach", k_node_reach, lb, 256, s, (const u64*)sv.lower_mask, (i64)src->n1, 64, op, oi.m,
               lreach, lb, (const u64*)nullptr, (i64)0, (uint32_t*)nullptr);
      }
      launch("k_lower_mark", k_lower_mark, ceil_div(nL, 256), 256, s, (const int4*)sv.lower_origin,
             (const u64*)sv.lower_mask, (const uint32_t*)lreach, nL, op, oi.m, (const int32_t*)tile_of_cand,
             (const int32_t*)ts.d_num_tiles, ts.tile_child, ts.flags);
      // small batches: one launch, the table filled by its last workgroup (the
      // tile stage zeroed the counter); larger ones fill the table wide
      if (bounded) {
        tree_rank_tiles_last(ts, rank_ctr, cand_src, oi.m_src, s);
      } else {
        tree_rank_tiles(ts, s);
        fill_pair(cand_src, -1, nL * oi.m_src, oi.m_src, ts.cand_child, 0, 0, 64, ts.d_num_cands, s);
      }
      launch("k_lower_nbr", k_lower_nbr, ceil_div(nL, 256), 256, s, (const int4*)sv.lower_origin,
             (const u64*)sv.lower_mask, (const uint32_t*)lreach, nL, op, oi.m, oi.m_src, (const int32_t*)tile_of_cand,
             (const u64*)ts.tile_child, (const uint16_t*)ts.tile_prefix, (const int32_t*)ts.tile_lower_base,
             (const int32_t*)ts.d_num_tiles, (const int32_t*)ts.d_num_cands, lower_nbr, ts.cand_origin, cand_src,
             ts.flags);
    }
    // leaves: every candidate's 16^3 mask, its prefix table and packed count
    // (each candidate is written by exactly one wave or workgroup)
    if (op == TC_OP_REFINE) {
      launch("k_leaf_mark_lower", k_leaf_mark_lower, 2 * (i64)src->n1, 256, s, (const int4*)sv.leaf_origin,
             (const u64*)sv.leaf_mask, (const int32_t*)sv.lower_first, (const u64*)sv.lower_mask,
             (const uint16_t*)sv.lower_prefix, op, oi.m, (const int32_t*)lower_nbr, (const int32_t*)ts.d_num_cands,
             ts.cand_child, ts.cand_prefix, ts.cand_counts, ts.flags);
    } else if (op == TC_OP_COARSEN) {
      launch("k_mark_coarsen", k_mark_coarsen, ceil_div(nL, 4), 256, s, (const int32_t*)cand_src,
             (const int32_t*)ts.d_num_cands, (const u64*)sv.lower_mask, sv.n_lower, ts.cand_child, ts.cand_prefix,
             ts.cand_counts, ts.flags);
    } else if (nL > 0) {  // no source lowers: nothing to mark and every bbox is empty
      // one resident round of workgroups (a multiple of 8), each looping over its candidates
      const i64 resident = oi.lo < 0 && oi.hi > 0 ? mark_box_resident<-1, 1>()
                           : (oi.lo < 0 ? mark_box_resident<-1, 0>() : mark_box_resident<0, 1>());
      const i64 blocks = std::max<i64>(8, std::min(ceil_div(ts.cap_cands, 8), resident / 8) * 8);
      auto mark_box = oi.lo < 0 && oi.hi > 0 ? k_leaf_mark_box<-1, 1>
                      : (oi.lo < 0 ? k_leaf_mark_box<-1, 0> : k_leaf_mark_box<0, 1>);
      launch("k_leaf_mark_box", mark_box, blocks, 256, s, (const int32_t*)cand_src,
             (const int32_t*)ts.d_num_cands, B, (const tc_grid_header*)sv.headers,
             (const u64*)sv.lower_mask, (const uint16_t*)sv.lower_prefix, (const int32_t*)sv.lower_first,
             (const u64*)sv.leaf_mask, sv.n_lower, sv.n_leaf, ts.cand_child, ts.cand_prefix, ts.cand_counts,
             ts.flags);
    }
    ts.cand_counts_ready = true;
    // counts (small batches whose lower stage ran in one workgroup: inside the
    // node writer's launch below)
    // (exact layout: the one-workgroup counts stages write the readback words
    // straight into pinned host memory, the others leave them for a copy)
    const bool counted_writer = bounded && small_lowers && write_nodes_counted_fits(ts, B);
    const size_t rb_bytes = 4 * (4 + 3 * (size_t)B);
    int32_t* h_rb = bounded ? nullptr : static_cast<int32_t*>(pinned_staging(rb_bytes));
    bool rb_written = false;
    if (!counted_writer) rb_written = tree_counts(ts, B, s, h_rb);
    if (bounded) {  // capacity layout: allocated while the stages above run
      out = new_batch_capacity(B, nT, nL, L_cap, oa);
    } else {  // exact layout: counts first, then the allocation
      if (!rb_written) hip_check(hipMemcpyAsync(h_rb, ts.readback, rb_bytes, hipMemcpyDeviceToHost, s), "readback");
      hip_check(hipStreamSynchronize(s), "hipStreamSynchronize");
      check_pass_flags(h_rb[0]);
      out = new_batch(B, h_rb, oa);
      if (out->nl > 0 && sv.n_leaf == 0) throw Error(TC_ERR_INTERNAL, "pass: output leaves without source leaves");
    }
    // writers (launch bounds and scratch by the leaf count, or its capacity)
    const GridView ov = bounded ? make_view(out->buffer, out->layout, B, (int32_t)nT, (int32_t)nL, (int32_t)L_cap)
                                : out->view();
    const i64 L = ov.n_leaf;
    const int32_t* d_L = ts.readback + 3;  // the leaf count on the device
    Arena post(s);
    const size_t o_lc = post.reserve(4 * L);
    const size_t o_box = post.reserve(4 * L);
    const size_t o_bb = post.reserve(4 * 6 * (i64)B * bbox_replicas(B));
    const size_t o_part = post.reserve(8 * (ceil_div(L, gran) + 1));  // voxel sums per gather workgroup
    const size_t o_gvb = post.reserve(8 * ((i64)B + 1));
    const size_t o_inrun = post.reserve(4 * L);
    post.commit();
    int32_t* leaf_cand = post.at<int32_t>(o_lc);
    i64* vox_part = post.at<i64>(o_part);
    int32_t* leaf_inrun = post.at<int32_t>(o_inrun);
    if (counted_writer) {
      tree_write_nodes_counted(ts, ov, leaf_cand, s);
    } else {
      tree_write_nodes(ts, ov, leaf_cand, s);
    }
    if (op == TC_OP_REFINE || op == TC_OP_COARSEN) {
      const i64 lanes = op == TC_OP_REFINE ? 1 : 4;
      auto gather = op == TC_OP_REFINE ? k_leaf_gather<0> : k_leaf_gather<1>;
      launch("k_leaf_gather", gather, ceil_div(L * lanes, 256), 256, s, (const int4*)ov.leaf_origin,
             (const int32_t*)leaf_cand, d_L, L, (const int32_t*)cand_src, (const u64*)sv.lower_mask,
             (const uint16_t*)sv.lower_prefix, (const int32_t*)sv.lower_first, (const u64*)sv.leaf_mask, sv.n_lower,
             sv.n_leaf, (const int32_t*)ts.d_num_cands, ov.leaf_mask, ov.leaf_prefix, post.at<uint32_t>(o_box),
             leaf_inrun, vox_part, ts.flags);
    } else {
      // buffer loads when every array they read stays under 2 GiB
      const bool buf = (i64)sv.n_leaf * 64 < (1ll << 31) && (i64)sv.n_lower * 512 < (1ll << 31) &&
                       ts.cap_cands * 27 * 4 < (1ll << 31) && !debug_wide_loads();
      auto gather_box = oi.lo < 0 && oi.hi > 0 ? (buf ? k_leaf_gather_box<-1, 1, true> : k_leaf_gather_box<-1, 1, false>)
                        : oi.lo < 0 ? (buf ? k_leaf_gather_box<-1, 0, true> : k_leaf_gather_box<-1, 0, false>)
                                    : (buf ? k_leaf_gather_box<0, 1, true> : k_leaf_gather_box<0, 1, false>);
      launch("k_leaf_gather", gather_box, ceil_div(L * 4, 256), 256, s, (const int4*)ov.leaf_origin,
             (const int32_t*)leaf_cand, d_L, L, (const int32_t*)cand_src, (const u64*)sv.lower_mask,
             (const uint16_t*)sv.lower_prefix, (const int32_t*)sv.lower_first, (const u64*)sv.leaf_mask, sv.n_lower,
             sv.n_leaf, (const int32_t*)ts.d_num_cands, ov.leaf_mask, ov.leaf_prefix, post.at<uint32_t>(o_box),
             leaf_inrun, vox_part, ts.flags, (uint32_t)std::min<i64>(ts.cap_cands * 27 * 4, (1ll << 31) - 1));
    }
    // the gathers' consistency checks set bits in the flag word after the
    // counts: the finalize copies it into the batch's status word
    apply_debug_inject(ts.flags, s);
    // small batches: the finalize's workgroup 0 writes every header's counts and
    // the status word into pinned host memory (the pass's one readback); a deferred
    // pass keeps that memory with the batch and leaves the wait to resolve_counts
    const size_t hb = sizeof(tc_grid_header) * (size_t)B + 16;
    char* h = nullptr;
    if (bounded && defer) {
      out->hdr_host = pinned_block_take(hb, &out->hdr_host_cap);
      h = static_cast<char*>(out->hdr_host);
    } else if (bounded) {
      h = static_cast<char*>(pinned_staging(hb));
    }
    tree_finalize_leaves(ov, post.at<uint32_t>(o_box), leaf_inrun, vox_part, gran, post.at<i64>(o_gvb),
                         post.at<int32_t>(o_bb), (const int32_t*)ts.grid_info, ts.flags, d_L, s,
                         reinterpret_cast<int32_t*>(h));
    if (bounded && defer) {
      out->hdr_ev = pending_event_take(out->device);
      hip_check(hipEventRecord(out->hdr_ev, s), "hipEventRecord");
      out->hdr_pending = true;
    } else if (bounded) {
      hip_check(hipStreamSynchronize(s), "hipStreamSynchronize");
      check_pass_flags(*reinterpret_cast<const int32_t*>(h + sizeof(tc_grid_header) * (size_t)B));
      set_counts_from_headers(out, reinterpret_cast<const tc_grid_header*>(h));
    }
  } catch (...) {
    free_batch(out);
    throw;
  }
  return out;
}

}  // namespace tc
