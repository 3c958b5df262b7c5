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

__global__ void __launch_bounds__(256) k_voxel_grid(const i64* offsets, int32_t B, i64 n, int32_t* vgrid) {
  const i64 i = (i64)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  int32_t lo = 0, hi = B - 1;  // last g with offsets[g] <= i
  while (lo < hi) {
    const int32_t mid = lo + (hi - lo + 1) / 2;
    if (offsets[mid] <= i) lo = mid;
    else hi = mid - 1;
  }
  vgrid[i] = lo;
}

// Voxels that arrive together usually share their tile, lower and leaf, so the
// lanes of a wave first merge the bits they set in the same 64-bit word (up to
// kDedupRounds distinct words, found with ballots and shuffles, no memory
// traffic); then every group's leader issues one OR for the union, all groups
// at once. Lanes still waiting after kDedupRounds words OR their own bit. With
// kCheck the leaders first read their word and skip the atomic when the bits
// are already set: the words of tiles and lower nodes are shared by many waves
// and same-address device atomics serialize, whereas leaf words mostly receive
// new bits and are ORed without the read.
constexpr int kDedupRounds = 8;

__device__ __forceinline__ u64 wave_or_u64(u64 v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v |= __shfl_xor(v, d, kWave);
  return v;
}

template <bool kCheck>
__device__ __forceinline__ void wave_or_into(u64* word, u64 bits, bool active) {
  const int lane = threadIdx.x & (kWave - 1);
  u64 todo = __ballot(active);
  u64 mine = 0;  // the union this lane ORs, if it leads a group
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
  if (mine && (!kCheck || (*word & mine) != mine)) atomicOr((unsigned long long*)word, mine);
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
__device__ int32_t tile_probe(const int32_t* ijk, const int32_t* vgrid, i64 i, int32_t g, int32_t tx, int32_t ty,
                              int32_t tz, int32_t* table, i64 H, int32_t* flags) {
  i64 h = (i64)(tile_hash(g, tx, ty, tz) & (u64)(H - 1));
  for (i64 probe = 0; probe < H; ++probe) {
    int32_t e = __hip_atomic_load(&table[h], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (e < 0) {
      const int32_t old = atomicCAS(&table[h], -1, (int32_t)i);
      if (old < 0) return (int32_t)i;
      e = old;
    }
    if (vgrid[e] == g && (ijk[(i64)e * 3] >> 12) == tx && (ijk[(i64)e * 3 + 1] >> 12) == ty &&
        (ijk[(i64)e * 3 + 2] >> 12) == tz)
      return e;
    h = (h + 1) & (H - 1);
  }
  atomicOr(flags, 2);
  return (int32_t)i;
}

// Lanes of a wave that share a (grid, tile) probe once, through one leader.
__global__ void __launch_bounds__(256) k_hash_tiles(const int32_t* ijk, const int32_t* vgrid, i64 n, int32_t* table,
                                                    i64 H, int32_t* rep, int32_t* flags) {
  const i64 i = (i64)blockIdx.x * 256 + threadIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const bool in = i < n;
  int32_t g = 0, tx = 0, ty = 0, tz = 0;
  if (in) {
    g = vgrid[i];
    tx = ijk[i * 3] >> 12;
    ty = ijk[i * 3 + 1] >> 12;
    tz = ijk[i * 3 + 2] >> 12;
  }
  int32_t mine = -1;
  u64 todo = __ballot(in);
  for (int round = 0; todo && round < kDedupRounds; ++round) {
    const int leader = __builtin_ctzll(todo);
    const int32_t lg = __shfl(g, leader, kWave), lx = __shfl(tx, leader, kWave), ly = __shfl(ty, leader, kWave),
                  lz = __shfl(tz, leader, kWave);
    const bool same = ((todo >> lane) & 1ull) && g == lg && tx == lx && ty == ly && tz == lz;
    const u64 sm = __ballot(same);
    int32_t r = -1;
    if (lane == leader) r = tile_probe(ijk, vgrid, i, g, tx, ty, tz, table, H, flags);
    r = __shfl(r, leader, kWave);
    if (same) mine = r;
    todo &= ~sm;
  }
  if ((todo >> lane) & 1ull) mine = tile_probe(ijk, vgrid, i, g, tx, ty, tz, table, H, flags);
  if (in) rep[i] = mine;
}

__global__ void __launch_bounds__(256) k_rep_flags(const int32_t* rep, i64 n, int32_t* flag) {
  const i64 i = (i64)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  flag[i] = rep[i] == i ? 1 : 0;
}

__global__ void __launch_bounds__(256) k_tile_compact(const int32_t* ijk, const int32_t* vgrid, const int32_t* flag,
                                                      const int32_t* excl, i64 n, Key128* keys, uint32_t* vals) {
  const i64 i = (i64)blockIdx.x * 256 + threadIdx.x;
  if (i >= n || !flag[i]) return;
  const int32_t k = excl[i];
  const u64 g = (uint32_t)vgrid[i];
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
  const i64 i = (i64)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int32_t r = rep[i];
  const int32_t k = (r >= 0 && r < n) ? excl[r] : -1;
  const int32_t t = (k >= 0 && k < nt) ? rank_of[k] : -1;
  if (t < 0 || t >= nt) {
    atomicOr(flags, 2);
    vtile[i] = 0;
    return;
  }
  vtile[i] = t;
}

__global__ void __launch_bounds__(256) k_voxel_mark_lower(const int32_t* ijk, const int32_t* vtile, i64 n,
                                                          u64* tile_child) {
  const i64 i = (i64)blockIdx.x * 256 + threadIdx.x;
  const bool in = i < n;
  u64* word = tile_child;
  u64 b = 0;
  if (in) {
    const i64 t = vtile[i];
    const int kx = (ijk[i * 3] >> 7) & 31, ky = (ijk[i * 3 + 1] >> 7) & 31, kz = (ijk[i * 3 + 2] >> 7) & 31;
    const int bit = (kx * 32 + ky) * 32 + kz;
    word = &tile_child[t * 512 + (bit >> 6)];
    b = 1ull << (bit & 63);
  }
  wave_or_into<true>(word, b, in);
}

// All lanes stay active to the end of these kernels (no early return), so the
// wave-wide merges see every lane.
__global__ void __launch_bounds__(256) k_voxel_cand(const int32_t* ijk, const int32_t* vtile, i64 n,
                                                    const u64* tile_child, const uint16_t* tile_prefix,
                                                    const int32_t* tile_lower_base, int32_t nc, int32_t* vcand,
                                                    int4* cand_origin, u64* cand_child, int32_t* flags) {
  const i64 i = (i64)blockIdx.x * 256 + threadIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  bool ok = i < n;
  int32_t c = -1, x = 0, y = 0, z = 0;
  i64 t = 0;
  if (ok) {
    t = vtile[i];
    x = ijk[i * 3];
    y = ijk[i * 3 + 1];
    z = ijk[i * 3 + 2];
    const int bit = (((x >> 7) & 31) * 32 + ((y >> 7) & 31)) * 32 + ((z >> 7) & 31);
    const int w = bit >> 6, b = bit & 63;
    c = tile_lower_base[t] + tile_prefix[t * 512 + w] + popc64(tile_child[t * 512 + w] & ((1ull << b) - 1));
    if (c < 0 || c >= nc) {
      atomicOr(flags, 2);
      c = -1;
      ok = false;
    }
    vcand[i] = c;
  }
  // one lane per run of equal candidates writes the candidate's origin
  const int32_t cprev = __shfl_up(c, 1, kWave);
  if (ok && (lane == 0 || cprev != c))
    cand_origin[c] = make_int4((x >> 7) * 128, (y >> 7) * 128, (z >> 7) * 128, (int32_t)t);
  const int lb = (((x >> 3) & 15) * 16 + ((y >> 3) & 15)) * 16 + ((z >> 3) & 15);
  wave_or_into<true>(ok ? &cand_child[(i64)c * 64 + (lb >> 6)] : cand_child, ok ? 1ull << (lb & 63) : 0, ok);
}

__global__ void __launch_bounds__(256) k_voxel_leaf(const int32_t* ijk, const int32_t* vcand, i64 n,
                                                    const u64* cand_child, const uint16_t* cand_prefix,
                                                    const i64* cand_scan, i64 n_leaf, u64* leaf_mask) {
  const i64 i = (i64)blockIdx.x * 256 + threadIdx.x;
  bool ok = i < n;
  u64* word = leaf_mask;
  u64 bits = 0;
  if (ok) {
    const i64 c = vcand[i];
    if (c < 0) {
      ok = false;
    } else {
      const int32_t x = ijk[i * 3], y = ijk[i * 3 + 1], z = ijk[i * 3 + 2];
      const int lb = (((x >> 3) & 15) * 16 + ((y >> 3) & 15)) * 16 + ((z >> 3) & 15);
      const int w = lb >> 6, b = lb & 63;
      const i64 leaf = (i64)(cand_scan[c] & 0xffffffffll) + cand_prefix[c * 64 + w] +
                       popc64(cand_child[c * 64 + w] & ((1ull << b) - 1));
      if (leaf < 0 || leaf >= n_leaf) {  // consistency guard
        ok = false;
      } else {
        word = &leaf_mask[leaf * 8 + (x & 7)];
        bits = 1ull << ((y & 7) * 8 + (z & 7));
      }
    }
  }
  wave_or_into<false>(word, bits, ok);
}

static int32_t read_i32(const int32_t* d, hipStream_t s) {
  int32_t* h = static_cast<int32_t*>(pinned_staging(64));
  hip_check(hipMemcpyAsync(h, d, 4, hipMemcpyDeviceToHost, s), "readback");
  hip_check(hipStreamSynchronize(s), "hipStreamSynchronize");
  return h[0];
}

tc_grid_batch* build_from_ijk(const int32_t* d_ijk, const int64_t* h_off, int32_t B, const OutAlloc& oa) {
  hipStream_t s = oa.stream;
  const i64 N = h_off[B];
  i64 H = 1024;
  while (H < 2 * N) H <<= 1;

  // stage 1: voxel -> grid, tile representatives, unique tiles
  Arena a1(s);
  const size_t o_off = a1.reserve(8 * ((i64)B + 1));
  const size_t o_vg = a1.reserve(4 * N);
  const size_t o_tab = a1.reserve(4 * H);
  const size_t o_rep = a1.reserve(4 * N);
  const size_t o_flag = a1.reserve(4 * N);
  const size_t o_excl = a1.reserve(4 * (N + 1));
  const size_t o_vt = a1.reserve(4 * N);
  const size_t o_vc = a1.reserve(4 * N);
  const size_t o_rb = a1.reserve(4 * 4);
  a1.commit();
  i64* d_off = a1.at<i64>(o_off);
  int32_t* vgrid = a1.at<int32_t>(o_vg);
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
  launch("k_voxel_grid", k_voxel_grid, ceil_div(N, 256), 256, s, (const i64*)d_off, B, N, vgrid);
  launch("k_hash_tiles", k_hash_tiles, ceil_div(N, 256), 256, s, d_ijk, (const int32_t*)vgrid, N, table, H, rep,
         flags);
  launch("k_rep_flags", k_rep_flags, ceil_div(N, 256), 256, s, (const int32_t*)rep, N, flag);
  scan_excl_i32(flag, excl, N, nullptr, s);
  hip_check(hipStreamSynchronize(s), "hipStreamSynchronize");  // the pinned offsets are consumed
  const int32_t nt = read_i32(excl + N, s);
  if (read_i32(flags, s) & 2) throw Error(TC_ERR_INTERNAL, "from_ijk: tile hash overflow");

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
  launch("k_tile_compact", k_tile_compact, ceil_div(N, 256), 256, s, d_ijk, (const int32_t*)vgrid,
         (const int32_t*)flag, (const int32_t*)excl, N, keys, vals);
  sort_pairs_128(keys, vals, nt, tile_key_bits(B), s);
  launch("k_tile_rank_scatter", k_tile_rank_scatter, ceil_div(nt, 256), 256, s, (const Key128*)keys,
         (const uint32_t*)vals, (i64)nt, rank_of, ts.utile);
  launch("k_voxel_tile", k_voxel_tile, ceil_div(N, 256), 256, s, (const int32_t*)rep, (const int32_t*)excl,
         (const int32_t*)rank_of, N, nt, vtile, flags);
  tree_tile_ranges(ts, B, s);
  fill_u64(ts.tile_child, 0, 512 * (i64)nt, nullptr, 1, s);
  launch("k_voxel_mark_lower", k_voxel_mark_lower, ceil_div(N, 256), 256, s, d_ijk, (const int32_t*)vtile, N,
         ts.tile_child);
  tree_rank_tiles(ts, s);
  const int32_t nc = read_i32(ts.d_num_cands, s);
  if (read_i32(flags, s) & 2) throw Error(TC_ERR_INTERNAL, "from_ijk: tile ranking check failed");

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
  launch("k_voxel_cand", k_voxel_cand, ceil_div(N, 256), 256, s, d_ijk, (const int32_t*)vtile, N,
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
    launch("k_voxel_leaf", k_voxel_leaf, ceil_div(N, 256), 256, s, d_ijk, (const int32_t*)vcand, N,
           (const u64*)ts.cand_child, (const uint16_t*)ts.cand_prefix, (const i64*)ts.cand_scan, L,
           ov.leaf_mask);
    tree_leaf_stats(ov, post.at<uint32_t>(o_box), post.at<int32_t>(o_inrun), post.at<i64>(o_part), s);
    tree_finalize_leaves(ov, post.at<uint32_t>(o_box), post.at<int32_t>(o_inrun), post.at<i64>(o_part), 256,
                         post.at<i64>(o_gvb), post.at<int32_t>(o_bb), (const int32_t*)ts.grid_info, s);
  } catch (...) {
    free_batch(out);
    throw;
  }
  return out;
}

}  // namespace tc
