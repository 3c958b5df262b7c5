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

__global__ void __launch_bounds__(256) k_kernel_map(const int4* t_origin, const u64* t_mask, const i64* t_offset,
                                                    const tc_grid_header* t_hdr, i64 n_leaf, KmapSrc src,
                                                    KmapGeom gm, int32_t* out, int waves) {
  extern __shared__ int32_t s_dyn[];
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
  int32_t* vol = s_dyn + 512 + w * gm.wave_words;
  int32_t* s_voff = vol + R * R * R;
  int32_t* s_leaf = s_voff + 512;
  int32_t* s_lbase = s_leaf + kKmapMaxSlots;
  const int v_first = lane / KK, k_first = lane % KK;

  for (i64 l = (i64)blockIdx.x * waves + w; l < n_leaf; l += (i64)gridDim.x * waves) {  // uniform per wave
    const int4 o = t_origin[l];
    const int g = o.w;
    const u64 tword = t_mask[l * 8 + (lane >> 3)];
    const int trow = (int)((tword >> (8 * (lane & 7))) & 0xffull);
    const int tcnt = __popc(trow);
    const int tinc = wave_incl_scan(tcnt);
    const int n = __shfl(tinc, kWave - 1, kWave);
    const i64 jb = t_hdr[g].voxel_begin + t_offset[l];
    const int32_t ub = src.hdr[g].upper_begin, uc = src.hdr[g].upper_count;
    const i64 vb = src.hdr[g].voxel_begin;

    // region of source coordinates [A0, A1] and the volume's fine origin F0
    i64 F0[3], A0[3], A1[3];
    const int oc[3] = {o.x, o.y, o.z};
    bool empty = uc == 0;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
      if (gm.transposed) {
        F0[a] = (i64)oc[a] - gm.hi;
        A0[a] = -floor_div_s(-F0[a], S);                      // ceil(F0 / S)
        A1[a] = floor_div_s((i64)oc[a] + 7 - gm.lo, S);
      } else {
        F0[a] = (i64)S * oc[a] + gm.lo;
        A0[a] = F0[a];
        A1[a] = (i64)S * (oc[a] + 7) + gm.hi;
      }
      A0[a] = imax64(A0[a], (i64)INT32_MIN);
      A1[a] = imin64(A1[a], (i64)INT32_MAX);
      empty = empty || A0[a] > A1[a];
    }
    int L0[3] = {0, 0, 0}, W[3] = {0, 0, 0};
    if (!empty) {
#pragma unroll
      for (int a = 0; a < 3; ++a) {
        L0[a] = (int)(A0[a] >> 3);
        W[a] = (int)(A1[a] >> 3) - L0[a] + 1;
      }
    }
    const int nslots = W[0] * W[1] * W[2];  // <= kKmapMaxSlots for S <= 2, K <= 8

    // 1. the region's source leaves
    if (lane < nslots) {
      const int ix = lane / (W[1] * W[2]), iy = (lane / W[2]) % W[1], iz = lane % W[2];
      const int leaf = find_leaf(src, ub, uc, (L0[0] + ix) * 8, (L0[1] + iy) * 8, (L0[2] + iz) * 8);
      s_leaf[lane] = leaf;
      s_lbase[lane] = leaf >= 0 ? (int32_t)(vb + src.leaf_offset[leaf]) : 0;
    }
    const int R3 = R * R * R;
    for (int c = lane; c < R3; c += kWave) vol[c] = -1;
    // row voxel offsets: lane owns target row (x, y) = (lane >> 3, lane & 7)
    {
      const int m = gm.transposed ? 1 : S;  // the transposed conv's volume is at the target's resolution
      const int x = lane >> 3, y = lane & 7;
      int at = tinc - tcnt;
      int rest = trow;
      while (rest) {
        const int z = __builtin_ctz(rest);
        s_voff[at++] = ((m * x) * R + m * y) * R + m * z;
        rest &= rest - 1;
      }
    }
    wave_sync();

    // 2. scatter the region's active source voxels into the volume
    if (!empty) {
      const int m = gm.transposed ? S : 1;  // source coordinate -> volume coordinate scale
      const int nx = (int)(A1[0] - A0[0] + 1), ny = (int)(A1[1] - A0[1] + 1);
      const int zl0 = (int)(A0[2] >> 3), zl1 = (int)(A1[2] >> 3);
      for (int r = lane; r < nx * ny; r += kWave) {
        const int x = (int)(A0[0] + r / ny), y = (int)(A0[1] + r % ny);
        const int sx = (x >> 3) - L0[0], sy = (y >> 3) - L0[1];
        const i64 ux = (i64)m * x - F0[0], uy = (i64)m * y - F0[1];
        const int urow = (int)((ux * R + uy) * R);
        for (int zl = zl0; zl <= zl1; ++zl) {
          const int slot = (sx * W[1] + sy) * W[2] + (zl - L0[2]);
          const int leaf = s_leaf[slot];
          if (leaf < 0) continue;
          const u64 word = src.leaf_mask[(i64)leaf * 8 + (x & 7)];
          const int row = (int)((word >> (8 * (y & 7))) & 0xffull);
          // z bits of this leaf inside [A0z, A1z]
          const int lb = (int)(imax64(A0[2], (i64)zl * 8) - (i64)zl * 8);
          const int hb = (int)(imin64(A1[2], (i64)zl * 8 + 7) - (i64)zl * 8);
          int bits = row & ((2 << hb) - 1) & ~((1 << lb) - 1);
          if (!bits) continue;
          const u64 pre = src.leaf_prefix[leaf];
          const int wx = x & 7;
          const int before_word = wx == 0 ? 0 : (int)((pre >> (9 * (wx - 1))) & 511ull);
          const int before_row = __popcll(word & ((1ull << (8 * (y & 7))) - 1ull));
          const int32_t rank0 = s_lbase[slot] + before_word + before_row;
          while (bits) {
            const int z = __builtin_ctz(bits);
            const i64 uz = (i64)m * (zl * 8 + z) - F0[2];
            vol[urow + (int)uz] = rank0 + __popc(row & ((1 << z) - 1));
            bits &= bits - 1;
          }
        }
      }
    }
    wave_sync();

    // 3. rows out, K^3 entries each, coalesced
    int32_t* dst = out + jb * KK;
    const int P = n * KK;
    int v = v_first, k = k_first;
    for (int p = lane; p < P; p += kWave) {
      dst[p] = vol[s_voff[v] + s_koff[k]];
      v += gm.q64;
      k += gm.r64;
      if (k >= KK) {
        k -= KK;
        ++v;
      }
    }
    wave_sync();  // the next leaf reuses the wave's LDS
  }
}

}  // namespace

void kernel_map(const GridView& sv, const GridView& tv, int K, int S, int transposed, int32_t* out,
                hipStream_t s) {
  if (tv.n_leaf == 0) return;
  if (K < 1 || K > 8 || S < 1 || S > 2) throw Error(TC_ERR_UNSUPPORTED, "kernel_map: kernel/stride out of range");
  Arena arena(s);
  const size_t o_up = arena.reserve(sizeof(uint16_t) * 512 * (size_t)max(sv.n_upper, 1));
  arena.commit();
  uint16_t* upper_prefix = arena.at<uint16_t>(o_up);
  launch("k_upper_prefix", k_upper_prefix, sv.n_upper, 256, s, (const u64*)sv.upper_mask, upper_prefix);

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
  gm.wave_words = gm.R * gm.R * gm.R + 512 + 2 * kKmapMaxSlots;
  const size_t wave_bytes = 4 * (size_t)gm.wave_words;
  // waves per block while the block's LDS stays within 64 KiB
  int waves = 4;
  while (waves > 1 && 4 * 512 + waves * wave_bytes > 64 * 1024) waves >>= 1;
  const size_t lds = 4 * 512 + waves * wave_bytes;
  const i64 blocks = std::min<i64>(ceil_div(tv.n_leaf, waves), 1 << 20);

  KmapSrc src{(const tc_grid_header*)sv.headers, (const u64*)sv.upper_key, (const int32_t*)sv.upper_first,
              (const u64*)sv.upper_mask, (const uint16_t*)upper_prefix, (const int32_t*)sv.lower_first,
              (const u64*)sv.lower_mask, (const uint16_t*)sv.lower_prefix, (const u64*)sv.leaf_mask,
              (const u64*)sv.leaf_prefix, (const i64*)sv.leaf_offset};
  launch_lds("k_kernel_map", k_kernel_map, blocks, kWave * waves, lds, s, (const int4*)tv.leaf_origin,
             (const u64*)tv.leaf_mask, (const i64*)tv.leaf_offset, (const tc_grid_header*)tv.headers,
             (i64)tv.n_leaf, src, gm, out, waves);
}

}  // namespace tc
