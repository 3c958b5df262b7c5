// CPU oracle for batched generated-topology construction.
//
// TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or call
// this file; only the tests, the smoke check and the benchmark's CPU-baseline
// leg use it. It shares no code, header, table or helper with the HIP library.
//
// What it computes, member by member (set semantics, int64 arithmetic):
//   1. the op on the member's voxel set S
//        coarsen_f  : { floor(v / f) }                       f in {2,4,8}
//        refine_f   : { f*v + d : d in [0,f)^3 }             f in {2,4,8}
//        dilate     : { v + e : e in [-1,1]^3 }   (26-neighbour box dilation)
//        pad_neg    : { v + e : e in {-1,0}^3 }
//        pad_pos    : { v + e : e in {0,1}^3 }
//        k3s2 transpose : pad_neg(refine_2(S))
//        conv_s1 K  : { v + e : e in [-floor(K/2), floor((K-1)/2)]^3 }   K in [1,8]
//        conv_t_s1 K: { v + e : e in [-floor((K-1)/2), floor(K/2)]^3 }   K in [1,8]
//        identity   : S (a grid built directly from ijk)
//        masked refine f : refine_f({ v in S : keep[v] }), keep given per voxel
//                     in the canonical enumeration order of S (PR page, test
//                     plan: masked refine; the mask prunes voxels, then refines)
//      Source: "Batched leaf-mask topology construction for generated conv grids"
//      (PR page), sections 1 and 2; factors 4 and 8 are the closed forms of the
//      chained x2 passes described in section 1. The stride-1 kernel-K targets
//      (section 2, and K in {2,3,4,5} in the test plan) are the Minkowski sums
//      with the kernel's offset box O_K = [-floor((K-1)/2), floor(K/2)]^3: the
//      transposed conv scatters to S + O_K, the conv gathers from it, giving
//      S - O_K (reading: the pages do not fix which side an even kernel leans to).
//   2. the canonical order: root tiles by signed x-major tile coordinate (the
//      offset-shifted sort key), then the x-major upper-node child offset, then
//      the x-major lower-node child offset, then the x-major in-leaf bit index
//      (PR page section 1; test plan: elementwise ijk equality pins this order).
//   3. the tree derived from the ordered voxels: 8^3 leaves with 512-bit masks,
//      16^3-leaf lower nodes, 32^3-lower upper nodes (one root tile each), parent
//      links, first-child indices, per-grid counts, leaf voxel offsets and prefix
//      popcounts, per-grid bounding boxes (PR page section 1, last bullet).
//   4. kernel maps between two such batches: for every target voxel and kernel
//      offset, the index of the source voxel it reads (issue page, Measurements;
//      see oracle_kernel_map for the reading).
//
// Readings where the pages are silent (each is listed in the design notes):
//   * coarsening rounds toward -infinity; refinement anchors at f*v;
//   * no empty leaves or nodes are ever produced;
//   * in-leaf bit n = x*64 + y*8 + z (word x, bit y*8+z); lower child bit
//     (x*16+y)*16+z; upper child bit (x*32+y)*32+z;
//   * leaf voxel offset = 0-based running voxel count inside the grid;
//   * leaf prefix word packs seven 9-bit fields, field w-1 = voxels in words < w;
//   * lower prefix table entry w = active children in words < w;
//   * root key = (Tx+2^19)<<40 | (Ty+2^19)<<20 | (Tz+2^19), T = floor(c/4096);
//   * empty grid bbox = (INT32_MAX)^3 .. (INT32_MIN)^3;
//   * any output coordinate outside int32 rejects the whole call (status 2).
#include <algorithm>
#include <array>
#include <atomic>
#include <map>
#include <cstdint>
#include <cstring>
#include <new>
#include <system_error>
#include <thread>
#include <vector>

namespace {

using i64 = int64_t;
using u64 = uint64_t;

enum Op { OP_IDENTITY = 0, OP_COARSEN = 1, OP_REFINE = 2, OP_DILATE = 3,
          OP_PAD_NEG = 4, OP_PAD_POS = 5, OP_CONV_T_K3S2 = 6, OP_CONV_S1 = 7, OP_CONV_T_S1 = 8 };

enum Status { ST_OK = 0, ST_INVALID = 1, ST_OVERFLOW = 2, ST_NOMEM = 3 };

i64 floordiv(i64 a, i64 b) {
  i64 q = a / b;
  if ((a % b != 0) && ((a < 0) != (b < 0))) --q;
  return q;
}
i64 floormod(i64 a, i64 b) { return a - floordiv(a, b) * b; }

struct Vox { i64 x, y, z; };

// The canonical position of a voxel, compared lexicographically:
// (tile x,y,z) (upper child x,y,z) (lower child x,y,z) (in-leaf x,y,z).
using Key = std::array<i64, 12>;

Key canonical_key(const Vox& v) {
  const i64 c[3] = {v.x, v.y, v.z};
  Key k{};
  for (int a = 0; a < 3; ++a) {
    k[a] = floordiv(c[a], 4096);
    k[3 + a] = floormod(floordiv(c[a], 128), 32);
    k[6 + a] = floormod(floordiv(c[a], 8), 16);
    k[9 + a] = floormod(c[a], 8);
  }
  return k;
}

Vox voxel_of_key(const Key& k) {
  i64 c[3];
  for (int a = 0; a < 3; ++a) c[a] = k[a] * 4096 + k[3 + a] * 128 + k[6 + a] * 8 + k[9 + a];
  return {c[0], c[1], c[2]};
}

bool in_int32(i64 c) { return c >= INT32_MIN && c <= INT32_MAX; }

// Applies the op to one member's voxels (duplicates allowed in the output).
bool apply_op(int op, int factor, const std::vector<Vox>& in, std::vector<Vox>& out) {
  out.clear();
  auto box = [&](int lo, int hi, const std::vector<Vox>& src) {
    for (const Vox& v : src)
      for (int ex = lo; ex <= hi; ++ex)
        for (int ey = lo; ey <= hi; ++ey)
          for (int ez = lo; ez <= hi; ++ez) out.push_back({v.x + ex, v.y + ey, v.z + ez});
  };
  switch (op) {
    case OP_IDENTITY: out = in; break;
    case OP_COARSEN:
      for (const Vox& v : in)
        out.push_back({floordiv(v.x, factor), floordiv(v.y, factor), floordiv(v.z, factor)});
      break;
    case OP_REFINE:
      for (const Vox& v : in)
        for (int dx = 0; dx < factor; ++dx)
          for (int dy = 0; dy < factor; ++dy)
            for (int dz = 0; dz < factor; ++dz)
              out.push_back({v.x * factor + dx, v.y * factor + dy, v.z * factor + dz});
      break;
    case OP_DILATE: box(-1, 1, in); break;
    case OP_PAD_NEG: box(-1, 0, in); break;
    case OP_PAD_POS: box(0, 1, in); break;
    case OP_CONV_T_K3S2: {
      std::vector<Vox> fine;
      for (const Vox& v : in)
        for (int dx = 0; dx < 2; ++dx)
          for (int dy = 0; dy < 2; ++dy)
            for (int dz = 0; dz < 2; ++dz) fine.push_back({v.x * 2 + dx, v.y * 2 + dy, v.z * 2 + dz});
      box(-1, 0, fine);
      break;
    }
    case OP_CONV_S1: box(-(factor / 2), (factor - 1) / 2, in); break;
    case OP_CONV_T_S1: box(-((factor - 1) / 2), factor / 2, in); break;
    default: return false;
  }
  for (const Vox& v : out)
    if (!in_int32(v.x) || !in_int32(v.y) || !in_int32(v.z)) return false;
  return true;
}

int popcount64(u64 w) {
  int n = 0;
  for (int b = 0; b < 64; ++b) n += (int)((w >> b) & 1u);
  return n;
}

}  // namespace

// Result arrays, laid out like the fields the library exposes so that the tests
// can compare them element by element.
struct oracle_result {
  int32_t B = 0;
  std::vector<i64> headers;        // [B][16], see oracle_field_header
  std::vector<int32_t> upper_origin;  // [N2][4] x, y, z, grid
  std::vector<u64> upper_key;         // [N2]
  std::vector<int32_t> upper_first;   // [N2] index of first lower child
  std::vector<u64> upper_mask;        // [N2][512]
  std::vector<int32_t> lower_origin;  // [N1][4] x, y, z, parent upper
  std::vector<int32_t> lower_first;   // [N1] index of first leaf child
  std::vector<u64> lower_mask;        // [N1][64]
  std::vector<uint16_t> lower_prefix; // [N1][64]
  std::vector<int32_t> leaf_origin;   // [L][4] x, y, z, grid
  std::vector<int32_t> leaf_parent;   // [L]
  std::vector<u64> leaf_mask;         // [L][8]
  std::vector<u64> leaf_prefix;       // [L]
  std::vector<i64> leaf_offset;       // [L]
  std::vector<int32_t> ijk;           // [V][3]
};

extern "C" {

// Field ids for oracle_size / oracle_copy.
enum {
  ORACLE_HEADERS = 0, ORACLE_UPPER_ORIGIN, ORACLE_UPPER_KEY, ORACLE_UPPER_FIRST,
  ORACLE_UPPER_MASK, ORACLE_LOWER_ORIGIN, ORACLE_LOWER_FIRST, ORACLE_LOWER_MASK,
  ORACLE_LOWER_PREFIX, ORACLE_LEAF_ORIGIN, ORACLE_LEAF_PARENT, ORACLE_LEAF_MASK,
  ORACLE_LEAF_PREFIX, ORACLE_LEAF_OFFSET, ORACLE_IJK, ORACLE_NUM_FIELDS
};

// Builds the op's output for a batch of B members given as int32 ijk rows and
// int64 member offsets. Returns 0 on success, 1 for invalid arguments, 2 when an
// output coordinate leaves int32 (no result then), 3 when memory runs out.
int oracle_build(int op, int factor, const int32_t* ijk, const int64_t* offsets, int32_t B,
                 oracle_result** out) {
  if (!out) return ST_INVALID;
  *out = nullptr;
  if (B < 1 || !offsets) return ST_INVALID;
  if (offsets[0] != 0) return ST_INVALID;
  for (int g = 0; g < B; ++g)
    if (offsets[g + 1] < offsets[g]) return ST_INVALID;
  if (offsets[B] > 0 && !ijk) return ST_INVALID;
  const bool pow2 = factor == 2 || factor == 4 || factor == 8;
  switch (op) {
    case OP_COARSEN: case OP_REFINE: if (!pow2) return ST_INVALID; break;
    case OP_CONV_T_K3S2: if (factor != 2) return ST_INVALID; break;
    case OP_IDENTITY: case OP_DILATE: case OP_PAD_NEG: case OP_PAD_POS:
      if (factor != 1) return ST_INVALID;
      break;
    case OP_CONV_S1: case OP_CONV_T_S1: if (factor < 1 || factor > 8) return ST_INVALID; break;
    default: return ST_INVALID;
  }
  oracle_result* r = new (std::nothrow) oracle_result();
  if (!r) return ST_NOMEM;
  try {
    r->B = B;
    r->headers.assign((size_t)B * 16, 0);
    i64 voxel_total = 0;
    for (int g = 0; g < B; ++g) {
      std::vector<Vox> in;
      for (i64 i = offsets[g]; i < offsets[g + 1]; ++i)
        in.push_back({ijk[3 * i], ijk[3 * i + 1], ijk[3 * i + 2]});
      std::vector<Vox> res;
      if (!apply_op(op, factor, in, res)) { delete r; return ST_OVERFLOW; }
      std::vector<Key> keys;
      keys.reserve(res.size());
      for (const Vox& v : res) keys.push_back(canonical_key(v));
      std::vector<Vox>().swap(res);
      std::sort(keys.begin(), keys.end());
      keys.erase(std::unique(keys.begin(), keys.end()), keys.end());

      i64* h = &r->headers[(size_t)g * 16];
      const i64 upper_begin = (i64)r->upper_key.size();
      const i64 lower_begin = (i64)r->lower_first.size();
      const i64 leaf_begin = (i64)r->leaf_parent.size();
      i64 bmin[3] = {INT32_MAX, INT32_MAX, INT32_MAX};
      i64 bmax[3] = {INT32_MIN, INT32_MIN, INT32_MIN};
      i64 nvox = 0;
      for (size_t i = 0; i < keys.size(); ++i) {
        const Key& k = keys[i];
        const bool new_upper = i == 0 || !std::equal(k.begin(), k.begin() + 3, keys[i - 1].begin());
        const bool new_lower = new_upper || !std::equal(k.begin(), k.begin() + 6, keys[i - 1].begin());
        const bool new_leaf = new_lower || !std::equal(k.begin(), k.begin() + 9, keys[i - 1].begin());
        if (new_upper) {
          r->upper_origin.insert(r->upper_origin.end(),
              {(int32_t)(k[0] * 4096), (int32_t)(k[1] * 4096), (int32_t)(k[2] * 4096), (int32_t)g});
          const u64 ux = (u64)(k[0] + (1 << 19)), uy = (u64)(k[1] + (1 << 19)), uz = (u64)(k[2] + (1 << 19));
          r->upper_key.push_back((ux << 40) | (uy << 20) | uz);
          r->upper_first.push_back((int32_t)r->lower_first.size());
          r->upper_mask.insert(r->upper_mask.end(), 512, 0);
        }
        const i64 upper_idx = (i64)r->upper_key.size() - 1;
        if (new_lower) {
          r->lower_origin.insert(r->lower_origin.end(),
              {(int32_t)(k[0] * 4096 + k[3] * 128), (int32_t)(k[1] * 4096 + k[4] * 128),
               (int32_t)(k[2] * 4096 + k[5] * 128), (int32_t)upper_idx});
          r->lower_first.push_back((int32_t)r->leaf_parent.size());
          r->lower_mask.insert(r->lower_mask.end(), 64, 0);
          const i64 bit = (k[3] * 32 + k[4]) * 32 + k[5];
          r->upper_mask[(size_t)upper_idx * 512 + bit / 64] |= (u64)1 << (bit % 64);
        }
        const i64 lower_idx = (i64)r->lower_first.size() - 1;
        if (new_leaf) {
          r->leaf_origin.insert(r->leaf_origin.end(),
              {(int32_t)(k[0] * 4096 + k[3] * 128 + k[6] * 8), (int32_t)(k[1] * 4096 + k[4] * 128 + k[7] * 8),
               (int32_t)(k[2] * 4096 + k[5] * 128 + k[8] * 8), (int32_t)g});
          r->leaf_parent.push_back((int32_t)lower_idx);
          r->leaf_mask.insert(r->leaf_mask.end(), 8, 0);
          r->leaf_offset.push_back(nvox);
          const i64 bit = (k[6] * 16 + k[7]) * 16 + k[8];
          r->lower_mask[(size_t)lower_idx * 64 + bit / 64] |= (u64)1 << (bit % 64);
        }
        const i64 leaf_idx = (i64)r->leaf_parent.size() - 1;
        const i64 n = k[9] * 64 + k[10] * 8 + k[11];
        r->leaf_mask[(size_t)leaf_idx * 8 + n / 64] |= (u64)1 << (n % 64);
        const Vox v = voxel_of_key(k);
        r->ijk.insert(r->ijk.end(), {(int32_t)v.x, (int32_t)v.y, (int32_t)v.z});
        const i64 c[3] = {v.x, v.y, v.z};
        for (int a = 0; a < 3; ++a) {
          bmin[a] = std::min(bmin[a], c[a]);
          bmax[a] = std::max(bmax[a], c[a]);
        }
        ++nvox;
      }
      h[0] = g;
      h[1] = B;
      h[2] = (i64)r->upper_key.size() - upper_begin;
      h[3] = (i64)r->lower_first.size() - lower_begin;
      h[4] = (i64)r->leaf_parent.size() - leaf_begin;
      h[5] = upper_begin;
      h[6] = lower_begin;
      h[7] = leaf_begin;
      h[8] = nvox;
      h[9] = voxel_total;
      for (int a = 0; a < 3; ++a) { h[10 + a] = bmin[a]; h[13 + a] = bmax[a]; }
      voxel_total += nvox;
    }
    // Lower prefix tables: entry w counts active children in words 0..w-1.
    const size_t n1 = r->lower_first.size();
    r->lower_prefix.assign(n1 * 64, 0);
    for (size_t l = 0; l < n1; ++l) {
      int run = 0;
      for (int w = 0; w < 64; ++w) {
        r->lower_prefix[l * 64 + w] = (uint16_t)run;
        run += popcount64(r->lower_mask[l * 64 + w]);
      }
    }
    // Leaf prefix words: field w-1 (bits 9(w-1) .. 9(w-1)+8) = voxels in words 0..w-1.
    const size_t nl = r->leaf_parent.size();
    r->leaf_prefix.assign(nl, 0);
    for (size_t l = 0; l < nl; ++l) {
      u64 packed = 0;
      u64 run = 0;
      for (int w = 1; w < 8; ++w) {
        run += (u64)popcount64(r->leaf_mask[l * 8 + w - 1]);
        packed |= run << (9 * (w - 1));
      }
      r->leaf_prefix[l] = packed;
    }
  } catch (const std::bad_alloc&) {
    delete r;
    return ST_NOMEM;
  }
  *out = r;
  return ST_OK;
}

// Member-parallel driver of oracle_build. Members never interact (every op
// acts on one member's voxel set), so each member is built on its own, as a
// batch of one, by `threads` host threads that take members in turn (threads
// <= 0: one per hardware thread). The per-member results are then concatenated
// in member order: grid ids and counts are set to the batch's, node indices
// (first children, parents) and header begins are shifted by the nodes of the
// members before, and each member's voxels follow the previous members' voxels.
// The arithmetic per member is oracle_build's own. Same statuses as oracle_build
// (the lowest member's failure is reported).
int oracle_build_threaded(int op, int factor, const int32_t* ijk, const int64_t* offsets, int32_t B,
                          int32_t threads, oracle_result** out) {
  if (!out) return ST_INVALID;
  *out = nullptr;
  if (B < 1 || !offsets || offsets[0] != 0) return ST_INVALID;
  for (int g = 0; g < B; ++g)
    if (offsets[g + 1] < offsets[g]) return ST_INVALID;
  if (offsets[B] > 0 && !ijk) return ST_INVALID;
  int nt = threads > 0 ? threads : (int)std::thread::hardware_concurrency();
  if (nt < 1) nt = 1;
  if (nt > B) nt = B;
  std::vector<oracle_result*> part((size_t)B, nullptr);
  std::vector<int> status((size_t)B, ST_OK);
  std::atomic<int> next{0};
  auto worker = [&]() {
    for (;;) {
      const int g = next.fetch_add(1);
      if (g >= B) return;
      const int64_t one[2] = {0, offsets[g + 1] - offsets[g]};
      status[(size_t)g] = oracle_build(op, factor, one[1] ? ijk + 3 * offsets[g] : nullptr, one, 1, &part[(size_t)g]);
    }
  };
  std::vector<std::thread> pool;
  try {
    pool.reserve((size_t)nt);
    for (int t = 1; t < nt; ++t) pool.emplace_back(worker);
  } catch (const std::exception&) {  // fewer threads than asked: the started ones and this one finish
  }
  worker();
  for (std::thread& t : pool) t.join();
  int st = ST_OK;
  for (int g = 0; g < B && st == ST_OK; ++g) st = status[(size_t)g];
  oracle_result* r = st == ST_OK ? new (std::nothrow) oracle_result() : nullptr;
  if (st == ST_OK && !r) st = ST_NOMEM;
  if (st == ST_OK) {
    try {
      r->B = B;
      i64 nu = 0, n1 = 0, nl = 0, nv = 0;
      for (int g = 0; g < B; ++g) {
        const oracle_result& m = *part[(size_t)g];
        const i64* mh = m.headers.data();
        r->headers.insert(r->headers.end(), mh, mh + 16);
        i64* h = &r->headers[r->headers.size() - 16];
        h[0] = g;
        h[1] = B;
        h[5] = nu;
        h[6] = n1;
        h[7] = nl;
        h[9] = nv;
        for (size_t i = 0; i < m.upper_key.size(); ++i) {
          r->upper_origin.insert(r->upper_origin.end(), {m.upper_origin[4 * i], m.upper_origin[4 * i + 1],
                                                         m.upper_origin[4 * i + 2], (int32_t)g});
          r->upper_first.push_back((int32_t)(m.upper_first[i] + n1));
        }
        r->upper_key.insert(r->upper_key.end(), m.upper_key.begin(), m.upper_key.end());
        r->upper_mask.insert(r->upper_mask.end(), m.upper_mask.begin(), m.upper_mask.end());
        for (size_t i = 0; i < m.lower_first.size(); ++i) {
          r->lower_origin.insert(r->lower_origin.end(), {m.lower_origin[4 * i], m.lower_origin[4 * i + 1],
                                                         m.lower_origin[4 * i + 2],
                                                         (int32_t)(m.lower_origin[4 * i + 3] + nu)});
          r->lower_first.push_back((int32_t)(m.lower_first[i] + nl));
        }
        r->lower_mask.insert(r->lower_mask.end(), m.lower_mask.begin(), m.lower_mask.end());
        r->lower_prefix.insert(r->lower_prefix.end(), m.lower_prefix.begin(), m.lower_prefix.end());
        for (size_t i = 0; i < m.leaf_parent.size(); ++i) {
          r->leaf_origin.insert(r->leaf_origin.end(), {m.leaf_origin[4 * i], m.leaf_origin[4 * i + 1],
                                                       m.leaf_origin[4 * i + 2], (int32_t)g});
          r->leaf_parent.push_back((int32_t)(m.leaf_parent[i] + n1));
        }
        r->leaf_mask.insert(r->leaf_mask.end(), m.leaf_mask.begin(), m.leaf_mask.end());
        r->leaf_prefix.insert(r->leaf_prefix.end(), m.leaf_prefix.begin(), m.leaf_prefix.end());
        r->leaf_offset.insert(r->leaf_offset.end(), m.leaf_offset.begin(), m.leaf_offset.end());
        r->ijk.insert(r->ijk.end(), m.ijk.begin(), m.ijk.end());
        nu += (i64)m.upper_key.size();
        n1 += (i64)m.lower_first.size();
        nl += (i64)m.leaf_parent.size();
        nv += mh[8];
        delete part[(size_t)g];
        part[(size_t)g] = nullptr;
      }
    } catch (const std::bad_alloc&) {
      delete r;
      r = nullptr;
      st = ST_NOMEM;
    }
  }
  for (oracle_result* m : part) delete m;
  *out = r;
  return st;
}

// Number of elements (not bytes) of a field.
int64_t oracle_size(const oracle_result* r, int field) {
  if (!r) return -1;
  switch (field) {
    case ORACLE_HEADERS: return (int64_t)r->headers.size();
    case ORACLE_UPPER_ORIGIN: return (int64_t)r->upper_origin.size();
    case ORACLE_UPPER_KEY: return (int64_t)r->upper_key.size();
    case ORACLE_UPPER_FIRST: return (int64_t)r->upper_first.size();
    case ORACLE_UPPER_MASK: return (int64_t)r->upper_mask.size();
    case ORACLE_LOWER_ORIGIN: return (int64_t)r->lower_origin.size();
    case ORACLE_LOWER_FIRST: return (int64_t)r->lower_first.size();
    case ORACLE_LOWER_MASK: return (int64_t)r->lower_mask.size();
    case ORACLE_LOWER_PREFIX: return (int64_t)r->lower_prefix.size();
    case ORACLE_LEAF_ORIGIN: return (int64_t)r->leaf_origin.size();
    case ORACLE_LEAF_PARENT: return (int64_t)r->leaf_parent.size();
    case ORACLE_LEAF_MASK: return (int64_t)r->leaf_mask.size();
    case ORACLE_LEAF_PREFIX: return (int64_t)r->leaf_prefix.size();
    case ORACLE_LEAF_OFFSET: return (int64_t)r->leaf_offset.size();
    case ORACLE_IJK: return (int64_t)r->ijk.size();
    default: return -1;
  }
}

// Copies a field into dst (which must hold oracle_size(field) elements).
int oracle_copy(const oracle_result* r, int field, void* dst) {
  if (!r || !dst) return ST_INVALID;
  auto cp = [&](const auto& v) {
    if (!v.empty()) std::memcpy(dst, v.data(), v.size() * sizeof(v[0]));
    return (int)ST_OK;
  };
  switch (field) {
    case ORACLE_HEADERS: return cp(r->headers);
    case ORACLE_UPPER_ORIGIN: return cp(r->upper_origin);
    case ORACLE_UPPER_KEY: return cp(r->upper_key);
    case ORACLE_UPPER_FIRST: return cp(r->upper_first);
    case ORACLE_UPPER_MASK: return cp(r->upper_mask);
    case ORACLE_LOWER_ORIGIN: return cp(r->lower_origin);
    case ORACLE_LOWER_FIRST: return cp(r->lower_first);
    case ORACLE_LOWER_MASK: return cp(r->lower_mask);
    case ORACLE_LOWER_PREFIX: return cp(r->lower_prefix);
    case ORACLE_LEAF_ORIGIN: return cp(r->leaf_origin);
    case ORACLE_LEAF_PARENT: return cp(r->leaf_parent);
    case ORACLE_LEAF_MASK: return cp(r->leaf_mask);
    case ORACLE_LEAF_PREFIX: return cp(r->leaf_prefix);
    case ORACLE_LEAF_OFFSET: return cp(r->leaf_offset);
    case ORACLE_IJK: return cp(r->ijk);
    default: return ST_INVALID;
  }
}

void oracle_free(oracle_result* r) { delete r; }

// Masked refine: keep[j] (one byte per voxel, non-zero keeps) refers to the j-th
// voxel of the batch in canonical enumeration order (members in order, each
// member's distinct voxels sorted by canonical key). The kept voxels of every
// member are refined by `factor` (2, 4 or 8). Same statuses as oracle_build.
int oracle_build_masked_refine(int factor, const int32_t* ijk, const int64_t* offsets, int32_t B,
                               const uint8_t* keep, int64_t n_keep, oracle_result** out) {
  if (!out) return ST_INVALID;
  *out = nullptr;
  if (B < 1 || !offsets || offsets[0] != 0) return ST_INVALID;
  for (int g = 0; g < B; ++g)
    if (offsets[g + 1] < offsets[g]) return ST_INVALID;
  if (offsets[B] > 0 && !ijk) return ST_INVALID;
  try {
    std::vector<int32_t> kept_ijk;
    std::vector<int64_t> kept_off(1, 0);
    i64 j = 0;  // running index in the canonical enumeration
    for (int g = 0; g < B; ++g) {
      std::vector<std::pair<Key, Vox>> m;
      for (i64 i = offsets[g]; i < offsets[g + 1]; ++i) {
        const Vox v{ijk[3 * i], ijk[3 * i + 1], ijk[3 * i + 2]};
        m.push_back({canonical_key(v), v});
      }
      std::sort(m.begin(), m.end(), [](const std::pair<Key, Vox>& a, const std::pair<Key, Vox>& b) {
        return a.first < b.first;
      });
      m.erase(std::unique(m.begin(), m.end(),
                          [](const std::pair<Key, Vox>& a, const std::pair<Key, Vox>& b) { return a.first == b.first; }),
              m.end());
      for (const auto& kv : m) {
        if (j >= n_keep || !keep) return ST_INVALID;  // fewer flags than voxels
        if (keep[j])
          kept_ijk.insert(kept_ijk.end(), {(int32_t)kv.second.x, (int32_t)kv.second.y, (int32_t)kv.second.z});
        ++j;
      }
      kept_off.push_back((int64_t)(kept_ijk.size() / 3));
    }
    if (j != n_keep) return ST_INVALID;  // more flags than voxels
    return oracle_build(OP_REFINE, factor, kept_ijk.empty() ? nullptr : kept_ijk.data(), kept_off.data(), B, out);
  } catch (const std::bad_alloc&) {
    return ST_NOMEM;
  }
}


// Kernel map between a source and a target batch with the same member count.
// The issue page ("Generated-topology grid construction dominates per-iteration
// ConvolutionPlan cost", Measurements) names two kernel-map builds of a plan: a
// k3 s1 map on one topology and the k2s2 transposed-conv map. It gives neither
// their layout nor their offset order; reading: one row per target voxel, one
// column per kernel offset d in O_K^3 with O_K = [-floor((K-1)/2), floor(K/2)]
// (the offset box of the kernel-K targets above), columns x-major over d. For
// target voxel o of member g the entry is the index of the source voxel of
// member g at
//   conv:            S*o + d
//   transposed conv: (o - d) / S   when S divides every component of o - d,
// or -1 when there is none. Both batches are given as their canonical
// enumerations (ijk rows, member offsets); an index is a row of src_ijk.
// Returns 1 for invalid arguments, 2 when a source index would leave int32.
int oracle_kernel_map(const int32_t* src_ijk, const int64_t* src_off, const int32_t* dst_ijk,
                      const int64_t* dst_off, int32_t B, int K, int S, int transposed, int32_t* out) {
  if (B < 1 || !src_off || !dst_off || K < 1 || K > 8 || S < 1 || (transposed != 0 && transposed != 1))
    return ST_INVALID;
  if (src_off[0] != 0 || dst_off[0] != 0) return ST_INVALID;
  for (int g = 0; g < B; ++g)
    if (src_off[g + 1] < src_off[g] || dst_off[g + 1] < dst_off[g]) return ST_INVALID;
  if ((src_off[B] > 0 && !src_ijk) || (dst_off[B] > 0 && (!dst_ijk || !out))) return ST_INVALID;
  if (src_off[B] > (i64)INT32_MAX) return ST_OVERFLOW;
  const i64 lo = -((K - 1) / 2);
  const i64 kk = (i64)K * K * K;
  try {
    for (int g = 0; g < B; ++g) {
      std::map<std::array<i64, 3>, i64> index;  // this member's source voxels
      for (i64 i = src_off[g]; i < src_off[g + 1]; ++i)
        index[{src_ijk[3 * i], src_ijk[3 * i + 1], src_ijk[3 * i + 2]}] = i;
      for (i64 j = dst_off[g]; j < dst_off[g + 1]; ++j) {
        const i64 o[3] = {dst_ijk[3 * j], dst_ijk[3 * j + 1], dst_ijk[3 * j + 2]};
        for (i64 k = 0; k < kk; ++k) {
          const i64 d[3] = {lo + k / (K * K), lo + (k / K) % K, lo + k % K};
          std::array<i64, 3> c{};
          bool exact = true;
          for (int a = 0; a < 3; ++a) {
            if (transposed) {
              const i64 q = o[a] - d[a];
              if (floormod(q, S) != 0) exact = false;
              c[a] = floordiv(q, S);
            } else {
              c[a] = (i64)S * o[a] + d[a];
            }
          }
          const auto it = exact ? index.find(c) : index.end();
          out[j * kk + k] = it == index.end() ? -1 : (int32_t)it->second;
        }
      }
    }
  } catch (const std::bad_alloc&) {
    return ST_NOMEM;
  }
  return ST_OK;
}

}  // extern "C"
