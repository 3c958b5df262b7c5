// Grid batch from float32 points: the points front-end of the same batched
// back-end (PR page "Batched leaf-mask topology construction for generated conv
// grids", Measurements, follow-ups: from_points beside from_ijk).
//
// Member g's point p lies at x = (p - origin_g) / voxel_size_g in index space,
// a correctly rounded float32 subtract and divide per axis. Mode 0 keeps the
// voxel whose centre is nearest, floor(x + 1/2) (a tie goes to the larger
// index); mode 1 keeps the 2^3 voxels floor(x) + {0,1}^3 around the point. The
// rows then go through the ijk front-end, so duplicates collapse there.
#include <cmath>
#include <cstring>
#include <vector>

#include "device.hpp"
#include "internal.hpp"

namespace tc {

namespace {

constexpr int kPtsLdsMembers = 4095;  // member offsets searched in LDS up to this many members
constexpr int32_t kPtsNonFinite = 1;  // flag bits
constexpr int32_t kPtsOverflow = 2;

__global__ void __launch_bounds__(256) k_points_to_ijk(const float* xyz, const i64* offsets, int32_t B, i64 n,
                                                       const float* vs_org, int mode, int32_t* ijk,
                                                       int32_t* flags) {
  __shared__ i64 s_off[kPtsLdsMembers + 1];
  const bool lds = B <= kPtsLdsMembers;  // uniform
  if (lds) {
    for (int k = threadIdx.x; k <= B; k += 256) s_off[k] = offsets[k];
    __syncthreads();
  }
  const i64* off = lds ? s_off : offsets;
  const i64 i = (i64)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;  // no barrier below
  int32_t lo = 0, hi = B - 1;  // member: last g with offsets[g] <= i
  while (lo < hi) {
    const int32_t mid = lo + (hi - lo + 1) / 2;
    if (off[mid] <= i) lo = mid;
    else hi = mid - 1;
  }
  const int32_t g = lo;
  int32_t v[3];
  bool non_finite = false, overflow = false;
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    const float x = __fdiv_rn(__fsub_rn(xyz[i * 3 + a], vs_org[g * 6 + 3 + a]), vs_org[g * 6 + a]);
    v[a] = 0;
    if (!isfinite(x)) {
      non_finite = true;
      continue;
    }
    const float f = mode == 0 ? floorf(__fadd_rn(x, 0.5f)) : floorf(x);
    // floats at or above 2^31 are out; below it they are at most 2^31 - 128, so
    // mode 1's + 1 stays inside int32 too
    if (!(f >= -2147483648.0f && f < 2147483648.0f)) {
      overflow = true;
      continue;
    }
    v[a] = (int32_t)f;
  }
  if (non_finite) atomicOr(flags, kPtsNonFinite);
  if (overflow) atomicOr(flags, kPtsOverflow);
  if (mode == 0) {
#pragma unroll
    for (int a = 0; a < 3; ++a) ijk[i * 3 + a] = v[a];
  } else {
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int a = 0; a < 3; ++a) ijk[(i * 8 + c) * 3 + a] = v[a] + ((c >> (2 - a)) & 1);
  }
}

}  // namespace

tc_grid_batch* build_from_points(const float* d_xyz, const int64_t* h_off, int32_t B, const float* h_voxel_size,
                                 const float* h_origin, int mode, const OutAlloc& oa) {
  hipStream_t s = oa.stream;
  const i64 N = h_off[B];
  const i64 rows = mode == 0 ? N : 8 * N;
  Arena a(s);
  const size_t o_off = a.reserve(8 * ((size_t)B + 1));
  const size_t o_vo = a.reserve(4 * 6 * (size_t)B);
  const size_t o_ijk = a.reserve(12 * (size_t)std::max<i64>(rows, 1));
  const size_t o_flag = a.reserve(4);
  a.commit();
  i64* d_off = a.at<i64>(o_off);
  float* d_vo = a.at<float>(o_vo);
  int32_t* d_ijk = a.at<int32_t>(o_ijk);
  int32_t* d_flag = a.at<int32_t>(o_flag);

  // member offsets and (voxel size, origin) pairs, staged through pinned memory
  const size_t off_bytes = 8 * ((size_t)B + 1), vo_bytes = 4 * 6 * (size_t)B;
  char* h_stage = static_cast<char*>(pinned_staging(off_bytes + vo_bytes + 64));
  std::memcpy(h_stage, h_off, off_bytes);
  float* vo = reinterpret_cast<float*>(h_stage + off_bytes);
  for (int32_t g = 0; g < B; ++g)
    for (int k = 0; k < 3; ++k) {
      vo[g * 6 + k] = h_voxel_size[g * 3 + k];
      vo[g * 6 + 3 + k] = h_origin[g * 3 + k];
    }
  hip_check(hipMemcpyAsync(d_off, h_stage, off_bytes, hipMemcpyHostToDevice, s), "points upload");
  hip_check(hipMemcpyAsync(d_vo, vo, vo_bytes, hipMemcpyHostToDevice, s), "points upload");
  fill_i32(d_flag, 0, 1, nullptr, 1, s);
  launch("k_points_to_ijk", k_points_to_ijk, ceil_div(N, 256), 256, s, (const float*)d_xyz, (const i64*)d_off, B, N,
         (const float*)d_vo, mode, d_ijk, d_flag);
  int32_t* h_flag = reinterpret_cast<int32_t*>(h_stage + off_bytes + vo_bytes);
  hip_check(hipMemcpyAsync(h_flag, d_flag, 4, hipMemcpyDeviceToHost, s), "points flag");
  hip_check(hipStreamSynchronize(s), "hipStreamSynchronize");  // also retires the uploads from pinned memory
  if (*h_flag & kPtsNonFinite) throw Error(TC_ERR_INVALID_ARG, "a point maps to a non-finite index coordinate");
  if (*h_flag & kPtsOverflow) throw Error(TC_ERR_OVERFLOW, "a point maps to an index outside int32");
  std::vector<int64_t> row_off(h_off, h_off + B + 1);
  if (mode == 1)
    for (auto& r : row_off) r *= 8;
  return build_from_ijk(d_ijk, row_off.data(), B, oa);
}

}  // namespace tc
