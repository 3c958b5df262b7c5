// Kernel maps between two grid batches.
//
// A convolution plan reads, for every output voxel and every kernel offset, one
// input voxel (issue page "Generated-topology grid construction dominates
// per-iteration ConvolutionPlan cost", Measurements: a k3 s1 map on one
// topology and the k2s2 transposed-conv map). The table here has one row per
// target voxel (canonical enumeration order) and one column per offset d in
// O_K^3, O_K = [-floor((K-1)/2), floor(K/2)], x-major; the entry is the
// batch-global enumeration index of the same member's source voxel at S*o + d
// (conv) or at (o - d)/S when that division is exact (transposed conv), else -1.
//
// One wave per target leaf. All rows of a leaf read a small box of source
// voxels (its region): S*[o, o+7] + O_K for the conv, and for the transposed
// conv the sources whose S-multiples fall into [o, o+7] - O_K. The wave
//   1. looks the region's source leaves up in the source tree (one lane each),
//   2. scatters the indices of the region's active source voxels into an LDS
//      volume that is -1 elsewhere (one lane per region row, ranks from the
//      leaf offset, prefix word and popcounts),
//   3. streams the leaf's rows out: entry (v, k) is volume[voff[v] + koff[k]],
//      where voff depends on the row's voxel only and koff on the offset only,
//      so consecutive lanes write consecutive int32 (coalesced stores).
// The volume is kept at the target's fine resolution for the transposed conv
// (a source voxel c lands at S*c), so both directions share step 3.
#include <mutex>

#include "device.hpp"
#include "internal.hpp"

namespace tc {

namespace {

struct KmapSrc {
  const tc_grid_header* hdr;
  const u64* upper_key;
  const int32_t* upper_first;
  const u64* upper_mask;
  const uint16_t* upper_prefix;  // [N2][512] active lowers in words < w
  const int32_t* lower_first;
  const u64* lower_mask;
  const uint16_t* lower_prefix;
  const u64* leaf_mask;
  const u64* leaf_prefix;
  const i64* leaf_offset;
};

struct KmapGeom {
  int K, S, transposed;
  int lo, hi;      // O_K = [lo, hi]
  int R;           // volume side: 7S + K (conv) or 7 + K (transposed conv)
  int KK;          // K^3 columns
  int q64, r64;    // 64 = q64 * KK + r64
  int vol_words;   // R^3 rounded up to a multiple of 4
  int wave_words;  // LDS words per wave
};

constexpr int kKmapMaxSlots = 64;  // source leaves per region (4 per axis at most)

// Exclusive per-word popcount prefix of every upper node's child mask, so that
// a lower node is found with one table read and one popcount.
__global__ void __launch_bounds__(256) k_upper_prefix(const u64* upper_mask, uint16_t* upper_prefix) {
  __shared__ int s_wave[256 / kWave];
  const i64 base = (i64)blockIdx.x * 512 + 2 * threadIdx.x;
  const int c0 = __popcll(upper_mask[base]);
  const int c1 = __popcll(upper_mask[base + 1]);
  int total;
  const int ex = block_excl_scan<int, 256>(c0 + c1, s_wave, total);
  upper_prefix[base] = (uint16_t)ex;
  upper_prefix[base + 1] = (uint16_t)(ex + c0);
}

// Leaf of one member whose origin is (x, y, z) (multiples of 8), or -1. The
// member's root tiles are upper nodes [ub, ub + uc), sorted by key.
__device__ int find_leaf(const KmapSrc& s, int32_t ub, int32_t uc, int x, int y, int z) {
  const u64 key = ((u64)((x >> 12) + (1 << 19)) << 40) | ((u64)((y >> 12) + (1 << 19)) << 20) |
                  (u64)((z >> 12) + (1 << 19));
  int a = ub, b = ub + uc;
  while (a < b) {
    const int mid = (a + b) >> 1;
    if (s.upper_key[mid] < key) a = mid + 1;
    else b = mid;
  }
  if (a >= ub + uc || s.upper_key[a] != key) return -1;
  const int ubit = ((((x >> 7) & 31) * 32 + ((y >> 7) & 31)) * 32) + ((z >> 7) & 31);
  const u64 uw = s.upper_mask[(i64)a * 512 + (ubit >> 6)];
  if (!((uw >> (ubit & 63)) & 1ull)) return -1;
  const int lower = s.upper_first[a] + s.upper_prefix[(i64)a * 512 + (ubit >> 6)] +
                    __popcll(uw & ((1ull << (ubit & 63)) - 1ull));
  const int lbit = ((((x >> 3) & 15) * 16 + ((y >> 3) & 15)) * 16) + ((z >> 3) & 15);
  const u64 lw = s.lower_mask[(i64)lower * 64 + (lbit >> 6)];
  if (!((lw >> (lbit & 63)) & 1ull)) return -1;
  return s.lower_first[lower] + s.lower_prefix[(i64)lower * 64 + (lbit >> 6)] +
         __popcll(lw & ((1ull << (lbit & 63)) - 1ull));
}

__device__ __forceinline__ i64 imax64(i64 a, i64 b) { return a > b ? a : b; }
__device__ __forceinline__ i64 imin64(i64 a, i64 b) { return a < b ? a : b; }
__device__ __forceinline__ i64 floor_div_s(i64 a, int S) { return S == 1 ? a : (a >> 1); }  // S in {1, 2}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Source-coordinate region [A0, A1] of target leaf origin o (clamped to int32),
// the volume's origin F0, and the window of source leaves: L0 + [0, W) per axis.
struct Region {
  i64 F0[3], A0[3], A1[3];
  int L0[3], W[3];
  bool empty;
};

__device__ __forceinline__ Region leaf_region(const int4& o, const KmapGeom& gm) {
  Region r;
  const int oc[3] = {o.x, o.y, o.z};
  r.empty = false;
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    if (gm.transposed) {
      r.F0[a] = (i64)oc[a] - gm.hi;
      r.A0[a] = -floor_div_s(-r.F0[a], gm.S);  // ceil(F0 / S)
      r.A1[a] = floor_div_s((i64)oc[a] + 7 - gm.lo, gm.S);
    } else {
      r.F0[a] = (i64)gm.S * oc[a] + gm.lo;
      r.A0[a] = r.F0[a];
      r.A1[a] = (i64)gm.S * (oc[a] + 7) + gm.hi;
    }
    r.A0[a] = imax64(r.A0[a], (i64)INT32_MIN);
    r.A1[a] = imin64(r.A1[a], (i64)INT32_MAX);
    r.empty = r.empty || r.A0[a] > r.A1[a];
  }
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    r.L0[a] = r.empty ? 0 : (int)(r.A0[a] >> 3);
    r.W[a] = r.empty ? 0 : (int)(r.A1[a] >> 3) - r.L0[a] + 1;
  }
  return r;
}

// One thread per (target leaf, window slot): the source leaf there and the
// batch-global index of its first voxel, or (-1, 0). `sm` slots per leaf. Also
// the batch-global index of every target leaf's first voxel (its first row).
__global__ void __launch_bounds__(256) k_kmap_slots(const int4* t_origin, const i64* t_offset,
                                                    const tc_grid_header* t_hdr, i64 n_leaf, KmapSrc src,
                                                    KmapGeom gm, int sm, int2* slots, i64* t_first) {
  const i64 t = (i64)blockIdx.x * 256 + threadIdx.x;
  if (t >= n_leaf * sm) return;
  const i64 l = t / sm;
  const int slot = (int)(t - l * sm);
  const int4 o = t_origin[l];
  if (slot == 0) t_first[l] = t_hdr[o.w].voxel_begin + t_offset[l];  // the leaf's first row
  const Region r = leaf_region(o, gm);
  int2 e = make_int2(-1, 0);
  if (slot < r.W[0] * r.W[1] * r.W[2]) {
    const tc_grid_header& h = src.hdr[o.w];
    const int ix = slot / (r.W[1] * r.W[2]), iy = (slot / r.W[2]) % r.W[1], iz = slot % r.W[2];
    const int leaf = find_leaf(src, h.upper_begin, h.upper_count, (r.L0[0] + ix) * 8, (r.L0[1] + iy) * 8,
                               (r.L0[2] + iz) * 8);
    if (leaf >= 0) e = make_int2(leaf, (int32_t)(h.voxel_begin + src.leaf_offset[leaf]));
  }
  slots[t] = e;
}

// Per-leaf inputs of the main kernel, loaded one leaf ahead.
struct LeafIn {
  int4 o;
  u64 tword;  // target mask word lane >> 3
  i64 first;  // batch-global index of the leaf's first row
  int2 slot;  // window slot `lane` (lanes below sm)
};

__device__ __forceinline__ LeafIn load_leaf(const int4* t_origin, const u64* t_mask, const i64* t_first,
                                            const int2* slots, int sm, i64 l, int lane) {
  LeafIn in;
  in.o = t_origin[l];
  in.tword = t_mask[l * 8 + (lane >> 3)];
  in.first = t_first[l];
  in.slot = slots[l * sm + min(lane, sm - 1)];  // lanes at or above sm ignore theirs
  return in;
}

// Main kernel. Per wave and target leaf, with the next leaf's inputs already in
// flight: lanes below sm load their slot's source leaf (8 mask words, prefix
// word) into LDS; the region's active voxels are ranked into the volume; the
// rows are streamed out. Volume coordinates are small and non-negative, so they
// are computed exactly in wrapping 32-bit arithmetic even where the region's
// origin lies outside int32.
__global__ void __launch_bounds__(256) k_kernel_map(const int4* t_origin, const u64* t_mask, const i64* t_first,
                                                    i64 n_leaf, KmapSrc src, KmapGeom gm, const int2* slots,
                                                    int sm, int32_t* out, int waves) {
  extern __shared__ __align__(16) int32_t s_dyn[];
  const int w = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int K = gm.K, S = gm.S, R = gm.R, KK = gm.KK;
  // column offsets inside the volume (shared by the block's waves)
  int32_t* s_koff = s_dyn;
  for (int k = threadIdx.x; k < KK; k += blockDim.x) {
    int d[3] = {k / (K * K), (k / K) % K, k % K};  // d - lo per axis
    if (gm.transposed)
#pragma unroll
      for (int a = 0; a < 3; ++a) d[a] = (K - 1) - d[a];  // hi - d
    s_koff[k] = (d[0] * R + d[1]) * R + d[2];
  }
  __syncthreads();
  // per-wave LDS: volume int32[vol_words] (R^3 rounded up to 4), slot masks
  // u64[sm][8], slot prefixes u64[sm], slot bases int32[sm], row offsets uint16[512]
  int32_t* vol = s_dyn + 512 + w * gm.wave_words;
  u64* s_smask = reinterpret_cast<u64*>(vol + gm.vol_words);
  u64* s_spre = s_smask + 8 * sm;
  int32_t* s_sbase = reinterpret_cast<int32_t*>(s_spre + sm);
  uint16_t* s_voff = reinterpret_cast<uint16_t*>(s_sbase + sm);
  // row streaming: up to 64 columns, lane owns column lane % KK of row lane / KK
  // (rows_per_it rows per store); wider rows take ceil(KK / 64) stores per row
  const int rows_per_it = KK <= kWave ? kWave / KK : 1;
  const bool col_lane = KK <= kWave && lane < rows_per_it * KK;
  const int my_row = KK <= kWave ? lane / KK : 0;
  int32_t koff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int k = KK <= kWave ? lane % KK : lane + kWave * j;
    koff[j] = k < KK ? s_koff[k] : 0;
  }

  i64 l = (i64)blockIdx.x * waves + w;
  const i64 stride = (i64)gridDim.x * waves;
  if (l >= n_leaf) return;  // uniform per wave; no block barrier below
  LeafIn cur = load_leaf(t_origin, t_mask, t_first, slots, sm, l, lane);
  for (; l < n_leaf; l += stride) {
    // this leaf's slot leaves, then the next leaf's inputs. The loads are
    // unconditional (absent slots read source leaf 0, clamped indices past the
    // end) so that no branch has to wait for them; selects come at the use.
    const bool have = lane < sm && cur.slot.x >= 0;
    const i64 sl = have ? cur.slot.x : 0;
    u64 m[8];
    const ulonglong2* mp = reinterpret_cast<const ulonglong2*>(src.leaf_mask + sl * 8);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const ulonglong2 v = mp[q];
      m[2 * q] = v.x;
      m[2 * q + 1] = v.y;
    }
    const u64 pre = src.leaf_prefix[sl];
    const i64 ln = l + stride;
    const LeafIn nxt = load_leaf(t_origin, t_mask, t_first, slots, sm, ln < n_leaf ? ln : l, lane);

    // row voxel offsets (lane owns target row (x, y) = (lane >> 3, lane & 7)) and the empty volume
    const uint32_t trow = (uint32_t)(cur.tword >> (8 * (lane & 7))) & 0xffu;
    const int tcnt = __popc(trow);
    const int tinc = wave_incl_scan(tcnt);
    const int n = __shfl(tinc, kWave - 1, kWave);
    {
      const int mv = gm.transposed ? 1 : S;  // the transposed conv's volume is at the target's resolution
      const int base = ((mv * (lane >> 3)) * R + mv * (lane & 7)) * R;
      int at = tinc - tcnt;
      uint32_t rest = trow;
      while (rest) {
        const int z = __builtin_ctz(rest);
        s_voff[at++] = (uint16_t)(base + mv * z);
        rest &= rest - 1;
      }
    }
    for (int c = lane; c < (gm.vol_words >> 2); c += kWave)
      reinterpret_cast<int4*>(vol)[c] = make_int4(-1, -1, -1, -1);
    if (lane < sm) {
#pragma unroll
      for (int q = 0; q < 8; ++q) s_smask[lane * 8 + q] = have ? m[q] : 0ull;
      s_spre[lane] = pre;
      s_sbase[lane] = cur.slot.y;
    }
    wave_sync();

    // scatter the region's active source voxels into the volume
    const Region r = leaf_region(cur.o, gm);
    if (!r.empty) {
      const uint32_t ms = gm.transposed ? (uint32_t)S : 1u;  // source coordinate -> volume coordinate scale
      const int ax0 = (int)r.A0[0], ay0 = (int)r.A0[1], az0 = (int)r.A0[2], az1 = (int)r.A1[2];
      const uint32_t fx = (uint32_t)r.F0[0], fy = (uint32_t)r.F0[1], fz = (uint32_t)r.F0[2];
      const int nx = (int)(r.A1[0] - r.A0[0] + 1), ny = (int)(r.A1[1] - r.A0[1] + 1);
      const int zl0 = az0 >> 3, nzl = (az1 >> 3) - zl0 + 1;
      const float inv_ny = 1.0f / (float)ny;
      for (int q = lane; q < nx * ny; q += kWave) {
        // q / ny for q < 2^11, ny <= 22: the float quotient is far from the next integer
        const int qx = (int)(((float)q + 0.5f) * inv_ny);
        const int x = ax0 + qx, y = ay0 + (q - qx * ny);
        const int sxy = (((x >> 3) - r.L0[0]) * r.W[1] + ((y >> 3) - r.L0[1])) * r.W[2];
        const uint32_t urow = ((ms * (uint32_t)x - fx) * (uint32_t)R + (ms * (uint32_t)y - fy)) * (uint32_t)R;
        const int wx = x & 7, by = 8 * (y & 7);
        for (int zi = 0; zi < nzl; ++zi) {
          const int zl = zl0 + zi;
          const int slot = sxy + zi;
          const u64 word = s_smask[slot * 8 + wx];
          const uint32_t row = (uint32_t)(word >> by) & 0xffu;
          // z bits of this leaf inside [az0, az1]
          const int lb = zi == 0 ? (az0 & 7) : 0;
          const int hb = zi == nzl - 1 ? (az1 & 7) : 7;
          uint32_t bits = row & ((2u << hb) - 1u) & ~((1u << lb) - 1u);
          if (!bits) continue;
          const int before_word = wx == 0 ? 0 : (int)((s_spre[slot] >> (9 * (wx - 1))) & 511ull);
          const int before_row = __popcll(word & ((1ull << by) - 1ull));
          const int32_t rank0 = s_sbase[slot] + before_word + before_row;
          const uint32_t uz0 = ms * (uint32_t)(zl * 8) - fz;
          while (bits) {
            const int z = __builtin_ctz(bits);
            vol[urow + uz0 + ms * (uint32_t)z] = rank0 + __popc(row & ((1u << z) - 1u));
            bits &= bits - 1;
          }
        }
      }
    }
    wave_sync();

    // rows out, K^3 entries each, coalesced
    int32_t* dst = out + cur.first * KK;
    if (KK <= kWave) {
      for (int v0 = 0; v0 < n; v0 += rows_per_it) {
        const int v = v0 + my_row;
        if (col_lane && v < n) dst[lane] = vol[s_voff[v] + koff[0]];
        dst += rows_per_it * KK;
      }
    } else {
      for (int v = 0; v < n; ++v) {
        const int vo = s_voff[v];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int k = lane + kWave * j;
          if (k < KK) dst[k] = vol[vo + koff[j]];
        }
        dst += KK;
      }
    }
    wave_sync();  // the next leaf reuses the wave's LDS
    cur = nxt;
  }
}

}  // namespace

static i64 host_floor_div(i64 a, i64 b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }

// Scratch of the no-allocation kernel map (tc_build_kernel_map_noalloc): one
// array per GPU, loaded with the library and held until the process ends. Its
// name is a host-side stand-in in host code; kernels get the device address
// that hipGetSymbolAddress returns for the current device.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_noalloc_mu;
char* g_noalloc_ptr[kMaxDevices] = {};
}  // namespace

char* noalloc_scratch(size_t* cap) {
  int dev = 0;
  hip_check(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) throw Error(TC_ERR_UNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lk(g_noalloc_mu);
  if (!g_noalloc_ptr[dev]) {  // once per device, with that device current
    void* p = nullptr;
    hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!p) throw Error(TC_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_noalloc_ptr[dev] = static_cast<char*>(p);
  }
  *cap = kNoAllocScratchBytes;
  return g_noalloc_ptr[dev];
}

// Geometry of a kernel map and its window slots per target leaf.
static KmapGeom kmap_geom(int K, int S, int transposed, int* slots_per_leaf) {
  KmapGeom gm;
  gm.K = K;
  gm.S = S;
  gm.transposed = transposed;
  gm.lo = -((K - 1) / 2);
  gm.hi = K / 2;
  gm.R = transposed ? 7 + K : 7 * S + K;
  gm.KK = K * K * K;
  gm.q64 = kWave / gm.KK;
  gm.r64 = kWave % gm.KK;
  // window slots per target leaf: the region's alignment to the leaf grid only
  // depends on the leaf origin modulo 16, so origins 0 and 8 give the maximum
  int sm = 0;
  for (int o = 0; o <= 8; o += 8) {
    i64 a0, a1;
    if (transposed) {
      a0 = -host_floor_div(-(o - gm.hi), S);
      a1 = host_floor_div(o + 7 - gm.lo, S);
    } else {
      a0 = (i64)S * o + gm.lo;
      a1 = (i64)S * (o + 7) + gm.hi;
    }
    const int w = (int)(host_floor_div(a1, 8) - host_floor_div(a0, 8) + 1);
    sm = std::max(sm, w * w * w);
  }
  if (sm > kKmapMaxSlots) throw Error(TC_ERR_INTERNAL, "kernel_map: window exceeds the slot table");
  // per wave: volume, slot masks and prefixes (18 words per slot), slot bases, 512 uint16 row offsets
  gm.vol_words = (gm.R * gm.R * gm.R + 3) & ~3;
  gm.wave_words = (gm.vol_words + 18 * sm + sm + 256 + 3) & ~3;  // 16-byte aligned waves
  *slots_per_leaf = sm;
  return gm;
}

// Scratch of one call, 256-byte aligned arrays: per source upper the popcount
// prefix of its child mask (uint16[512]); per (target leaf, window slot) the
// slot's source leaf and first voxel (int2); per target leaf its first row (int64).
struct KmapScratch {
  size_t up, slots, first, total;
};
static KmapScratch kmap_scratch(i64 n_upper, i64 n_leaf, int sm) {
  KmapScratch k{};
  k.up = 0;
  k.slots = align_up(k.up + sizeof(uint16_t) * 512 * (size_t)std::max<i64>(n_upper, 1));
  k.first = align_up(k.slots + sizeof(int2) * (size_t)n_leaf * sm);
  k.total = align_up(k.first + sizeof(i64) * (size_t)std::max<i64>(n_leaf, 1));
  return k;
}

size_t kernel_map_scratch_bytes(const GridView& sv, const GridView& tv, int K, int S, int transposed) {
  if (tv.n_leaf == 0 || sv.n_leaf == 0) return 0;
  if (K < 1 || K > 8 || S < 1 || S > 2) throw Error(TC_ERR_UNSUPPORTED, "kernel_map: kernel/stride out of range");
  int sm = 0;
  (void)kmap_geom(K, S, transposed, &sm);
  return kmap_scratch(sv.n_upper, tv.n_leaf, sm).total;
}

void kernel_map(const GridView& sv, const GridView& tv, int K, int S, int transposed, int32_t* out, i64 entries,
                hipStream_t s, char* scratch, size_t scratch_cap) {
  if (tv.n_leaf == 0) return;
  if (K < 1 || K > 8 || S < 1 || S > 2) throw Error(TC_ERR_UNSUPPORTED, "kernel_map: kernel/stride out of range");
  if (sv.n_leaf == 0) {  // no source voxel anywhere: every entry is -1
    fill_i32(out, -1, entries, nullptr, 1, s);
    return;
  }
  int sm = 0;
  const KmapGeom gm = kmap_geom(K, S, transposed, &sm);
  const KmapScratch lay = kmap_scratch(sv.n_upper, tv.n_leaf, sm);
  Arena arena(s);
  char* base = scratch;
  if (base) {
    if (lay.total > scratch_cap) throw Error(TC_ERR_INTERNAL, "kernel_map: scratch larger than the given buffer");
  } else {
    const size_t o = arena.reserve(lay.total);
    arena.commit();
    base = arena.at<char>(o);
  }
  uint16_t* upper_prefix = reinterpret_cast<uint16_t*>(base + lay.up);
  int2* slots = reinterpret_cast<int2*>(base + lay.slots);
  i64* t_first = reinterpret_cast<i64*>(base + lay.first);
  launch("k_upper_prefix", k_upper_prefix, sv.n_upper, 256, s, (const u64*)sv.upper_mask, upper_prefix);

  KmapSrc src{(const tc_grid_header*)sv.headers, (const u64*)sv.upper_key, (const int32_t*)sv.upper_first,
              (const u64*)sv.upper_mask, (const uint16_t*)upper_prefix, (const int32_t*)sv.lower_first,
              (const u64*)sv.lower_mask, (const uint16_t*)sv.lower_prefix, (const u64*)sv.leaf_mask,
              (const u64*)sv.leaf_prefix, (const i64*)sv.leaf_offset};
  launch("k_kmap_slots", k_kmap_slots, ceil_div((i64)tv.n_leaf * sm, 256), 256, s, (const int4*)tv.leaf_origin,
         (const i64*)tv.leaf_offset, (const tc_grid_header*)tv.headers, (i64)tv.n_leaf, src, gm, sm, slots,
         t_first);

  const size_t wave_bytes = 4 * (size_t)gm.wave_words;
  // waves per block while the block's LDS stays within 64 KiB
  int waves = 4;
  while (waves > 1 && 4 * 512 + waves * wave_bytes > 64 * 1024) waves >>= 1;
  const size_t lds = 4 * 512 + waves * wave_bytes;
  // one round of resident blocks (LDS and wave slots per CU decide how many);
  // each wave then walks many leaves, so the next leaf's inputs are always in flight
  const int cus = device_cu_count();
  const int per_cu = std::max(1, std::min(32 / waves, (int)((160 * 1024) / lds)));
  const i64 blocks = std::min<i64>(ceil_div(tv.n_leaf, waves), (i64)cus * per_cu);
  launch_lds("k_kernel_map", k_kernel_map, blocks, kWave * waves, lds, s, (const int4*)tv.leaf_origin,
             (const u64*)tv.leaf_mask, (const i64*)t_first, (i64)tv.n_leaf, src, gm, (const int2*)slots, sm, out,
             waves);
}

}  // namespace tc
