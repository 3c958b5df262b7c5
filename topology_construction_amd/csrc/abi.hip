// C ABI entry points (declared in include/topo.h): argument validation on the
// host, pass chaining for factors 4/8 and k3s2 transpose, batch ownership and
// error reporting. No exception crosses the boundary.
#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "internal.hpp"

namespace {

thread_local std::string t_last_error;

tc_status fail(tc_status s, const std::string& msg) {
  t_last_error = msg;
  return s;
}

template <typename F>
tc_status guarded(F&& f) {
  try {
    return f();
  } catch (const tc::Error& e) {
    return fail(e.status, e.what());
  } catch (const std::bad_alloc&) {
    return fail(TC_ERR_ALLOC, "host allocation failed");
  } catch (const std::exception& e) {
    return fail(TC_ERR_INTERNAL, e.what());
  }
}

int current_device() {
  int d = 0;
  tc::hip_check(hipGetDevice(&d), "hipGetDevice");
  return d;
}

}  // namespace

namespace tc {

// A batch handle with its buffer allocated for `layout` (counts still unset).
static tc_grid_batch* alloc_batch(int32_t B, const Layout& layout, const OutAlloc& oa) {
  tc_grid_batch* b = new tc_grid_batch();
  try {
    b->B = B;
    b->h_upper.assign(B, 0);
    b->h_lower.assign(B, 0);
    b->h_leaf.assign(B, 0);
    b->layout = layout;
    b->bytes = b->layout.total;
    const hipStream_t as = oa.transient || !oa.alloc_stream ? oa.stream : oa.alloc_stream;
    b->stream = as;
    b->device = current_device();
    if (oa.transient) {
      b->block = scratch_acquire(b->bytes, as);
      b->buffer = scratch_ptr(b->block);
    } else if (oa.alloc) {
      b->has_alloc = true;
      b->alloc = *oa.alloc;
      b->buffer = b->alloc.alloc(b->alloc.ctx, b->bytes, (void*)as);
      if (!b->buffer) throw Error(TC_ERR_ALLOC, "allocator returned NULL for " + std::to_string(b->bytes) + " bytes");
    } else {
      b->buffer = batch_buffer_take(b->bytes, as, &b->cap);
    }
  } catch (...) {
    delete b;
    throw;
  }
  return b;
}

tc_grid_batch* new_batch(int32_t B, const int32_t* rb, const OutAlloc& oa) {
  tc_grid_batch* b = alloc_batch(B, make_layout(B, rb[1], rb[2], rb[3]), oa);
  b->n2 = rb[1];
  b->n1 = rb[2];
  b->nl = rb[3];
  for (int32_t g = 0; g < B; ++g) {
    b->h_upper[g] = rb[4 + 3 * g];
    b->h_lower[g] = rb[4 + 3 * g + 1];
    b->h_leaf[g] = rb[4 + 3 * g + 2];
  }
  return b;
}

tc_grid_batch* new_batch_capacity(int32_t B, i64 n2_cap, i64 n1_cap, i64 nl_cap, const OutAlloc& oa) {
  return alloc_batch(B, make_layout(B, n2_cap, n1_cap, nl_cap), oa);
}

void set_counts_from_headers(tc_grid_batch* b, const tc_grid_header* h) {
  const int32_t B = b->B;
  i64 n2 = 0, n1 = 0, nl = 0, nv = 0;
  for (int32_t g = 0; g < B; ++g) {
    if (h[g].upper_begin != n2 || h[g].lower_begin != n1 || h[g].leaf_begin != nl || h[g].voxel_begin != nv ||
        h[g].upper_count < 0 || h[g].lower_count < 0 || h[g].leaf_count < 0 || h[g].voxel_count < 0)
      throw Error(TC_ERR_INTERNAL, "pass: inconsistent header counts");
    b->h_upper[g] = h[g].upper_count;
    b->h_lower[g] = h[g].lower_count;
    b->h_leaf[g] = h[g].leaf_count;
    n2 += h[g].upper_count;
    n1 += h[g].lower_count;
    nl += h[g].leaf_count;
    nv += h[g].voxel_count;
  }
  // the arrays sit at capacity offsets: the counts must fit the capacities
  const Layout& L = b->layout;
  if ((size_t)n2 * 16 > L.upper_key - L.upper_origin || (size_t)n1 * 16 > L.lower_first - L.lower_origin ||
      (size_t)nl * 16 > L.leaf_parent - L.leaf_origin)
    throw Error(TC_ERR_INTERNAL, "pass: counts above the output capacities");
  b->n2 = (int32_t)n2;
  b->n1 = (int32_t)n1;
  b->nl = (int32_t)nl;
  b->vox_total = nv;
  b->vox_known = true;
}

tc_grid_batch* copy_batch(const tc_grid_batch* src, const OutAlloc& oa) {
  tc_grid_batch* b = alloc_batch(src->B, src->layout, oa);
  b->n2 = src->n2;
  b->n1 = src->n1;
  b->nl = src->nl;
  b->h_upper = src->h_upper;
  b->h_lower = src->h_lower;
  b->h_leaf = src->h_leaf;
  try {
    // the same layout (exact or by capacities), so one copy moves every array
    hip_check(hipMemcpyAsync(b->buffer, src->buffer, src->bytes, hipMemcpyDeviceToDevice, oa.stream), "copy batch");
  } catch (...) {
    free_batch(b);
    throw;
  }
  return b;
}

void free_batch(tc_grid_batch* b) {
  if (!b) return;
  if (b->hdr_host) {  // headers still on their way land before the block is reused
    if (b->hdr_pending && b->hdr_ev) (void)hipEventSynchronize(b->hdr_ev);
    pinned_block_give(b->hdr_host, b->hdr_host_cap);
  }
  pending_event_give(b->device, b->hdr_ev);
  vox_slot_give(b->vox_slot);  // a copy still in flight is waited for by the slot's next taker
  if (b->block) {
    scratch_give_back(b->block, b->stream);
  } else if (b->buffer) {
    if (b->has_alloc) {
      if (b->alloc.free) b->alloc.free(b->alloc.ctx, b->buffer, b->bytes, (void*)b->stream);
    } else {
      batch_buffer_give(b->buffer, b->cap, b->device, b->stream);
    }
  }
  delete b;
}

static_assert(offsetof(tc_grid_header, voxel_begin) == offsetof(tc_grid_header, voxel_count) + 8,
              "voxel count and begin are read back as one 16-byte pair");

static void take_vox_slot(tc_grid_batch* b) {
  if (b->vox_slot >= 0) return;
  const VoxTicket t = vox_slot_take(b->device);
  b->vox_slot = t.slot;
  b->vox_h = t.h;
  b->vox_ev = t.ev;
}

namespace {
thread_local int32_t t_inject = 0;
thread_local bool t_wide_loads = false;
}
void debug_set_inject(int32_t bits) { t_inject = bits; }
void debug_set_wide_loads(bool on) { t_wide_loads = on; }
bool debug_wide_loads() { return t_wide_loads; }
void apply_debug_inject(int32_t* d_flags, hipStream_t s) {
  if (!t_inject) return;
  fill_i32(d_flags, t_inject, 1, nullptr, 1, s);  // testing: the writers "found" an inconsistency
  t_inject = 0;
}

// The last header's tail (voxel count and begin, bbox, reserved) and the status
// word after it are one contiguous 64-byte range, read back in one copy.
static_assert(sizeof(tc_grid_header) - offsetof(tc_grid_header, voxel_count) == 48, "header tail layout");
constexpr int kStatusWord = 6;  // int64 index of the status word in a 64-byte slot

static void apply_status(const tc_grid_batch* b) {
  if ((int32_t)b->vox_h[kStatusWord] != 0) b->status_bad = true;
}

void check_status(const tc_grid_batch* b) {
  if (b->vox_pending) {
    hip_check(hipEventSynchronize(b->vox_ev), "hipEventSynchronize");
    b->vox_total = b->vox_h[0] + b->vox_h[1];
    b->vox_known = true;
    b->vox_pending = false;
    apply_status(b);
  }
  if (b->status_bad)
    throw Error(TC_ERR_INTERNAL, "a device consistency check failed while this batch was written; its arrays are not valid");
}

// Queues the copy of the last member's header tail and the status word behind
// the builder's kernels (stream s) and records the slot's event, so that the
// first request for the total waits for that event instead of a new round trip.
static void queue_voxel_total(tc_grid_batch* b, hipStream_t s) {
  if (b->vox_known || b->B <= 0) return;
  take_vox_slot(b);
  const GridView v = b->view();
  hip_check(hipMemcpyAsync(b->vox_h, &v.headers[b->B - 1].voxel_count, 64, hipMemcpyDeviceToHost, s),
            "voxel total readback");
  hip_check(hipEventRecord(b->vox_ev, s), "hipEventRecord");
  b->vox_pending = true;
}

// Hands a finished batch to the caller with its voxel total queued; frees it if
// queueing fails.
static tc_grid_batch* finish_batch(tc_grid_batch* b, hipStream_t s) {
  try {
    queue_voxel_total(b, s);
  } catch (...) {
    free_batch(b);
    throw;
  }
  return b;
}

// The batch's voxel total: known, or waited for on its queued copy, or read
// back (into the pinned staging buffer, or with `pageable` into host stack
// memory, so that nothing is allocated).
static i64 read_voxel_total(const tc_grid_batch* b, hipStream_t s, bool pageable = false) {
  check_status(b);  // also takes the queued total
  if (b->vox_known) return b->vox_total;
  // nothing queued: the last header's tail and the status word, read back now
  int64_t stack_h[8];
  int64_t* h = pageable ? stack_h : static_cast<int64_t*>(pinned_staging(64));
  const GridView v = b->view();
  hip_check(hipMemcpyAsync(h, &v.headers[b->B - 1].voxel_count, 64, hipMemcpyDeviceToHost, s), "header readback");
  hip_check(hipStreamSynchronize(s), "hipStreamSynchronize");
  if ((int32_t)h[kStatusWord] != 0) b->status_bad = true;
  check_status(b);
  b->vox_total = h[0] + h[1];
  b->vox_known = true;
  return b->vox_total;
}

// The passes that build `op` with `factor`: a factor of 4 or 8 is two or three
// factor-2 passes, the k3s2 transpose is a refine and a negative pad, and a
// stride-1 convolution of kernel size k is the box [lo, hi] per axis made of
// dilates (one step on both sides) and pads (one step on one side).
tc_status op_passes(int32_t op, int32_t factor, std::vector<int>& passes, std::string& msg) {
  passes.clear();
  switch (op) {
    case TC_OP_COARSEN:
    case TC_OP_REFINE: {
      if (factor < 2) {
        msg = "refine/coarsen factor must be >= 2";
        return TC_ERR_INVALID_ARG;
      }
      if (factor != 2 && factor != 4 && factor != 8) {
        msg = "refine/coarsen factor must be 2, 4 or 8";
        return TC_ERR_UNSUPPORTED;
      }
      for (int f = factor; f > 1; f >>= 1) passes.push_back(op);
      return TC_OK;
    }
    case TC_OP_DILATE:
    case TC_OP_PAD_NEG:
    case TC_OP_PAD_POS:
      if (factor != 1) {
        msg = "box ops take factor 1";
        return TC_ERR_INVALID_ARG;
      }
      passes.push_back(op);
      return TC_OK;
    case TC_OP_CONV_T_K3S2:
      if (factor != 2) {
        msg = "k3s2 transpose takes factor 2";
        return TC_ERR_INVALID_ARG;
      }
      passes.push_back(TC_OP_REFINE);
      passes.push_back(TC_OP_PAD_NEG);
      return TC_OK;
    case TC_OP_CONV_S1:
    case TC_OP_CONV_T_S1: {
      if (factor < 1 || factor > 8) {
        msg = "kernel size must be in [1, 8]";
        return TC_ERR_INVALID_ARG;
      }
      const int o_lo = -((factor - 1) / 2), o_hi = factor / 2;
      const int lo = op == TC_OP_CONV_T_S1 ? o_lo : -o_hi, hi = op == TC_OP_CONV_T_S1 ? o_hi : -o_lo;
      const int both = std::min(-lo, hi);
      for (int i = 0; i < both; ++i) passes.push_back(TC_OP_DILATE);
      for (int i = 0; i < -lo - both; ++i) passes.push_back(TC_OP_PAD_NEG);
      for (int i = 0; i < hi - both; ++i) passes.push_back(TC_OP_PAD_POS);
      return TC_OK;
    }
    default:
      msg = "unknown op " + std::to_string(op);
      return TC_ERR_INVALID_ARG;
  }
}

}  // namespace tc

extern "C" {

int32_t tc_abi_version(void) { return TC_ABI_VERSION; }

const char* tc_status_string(tc_status s) {
  switch (s) {
    case TC_OK: return "ok";
    case TC_ERR_INVALID_ARG: return "invalid argument";
    case TC_ERR_OVERFLOW: return "int32 coordinate overflow";
    case TC_ERR_ALLOC: return "allocation failed";
    case TC_ERR_HIP: return "HIP runtime error";
    case TC_ERR_UNSUPPORTED: return "unsupported";
    case TC_ERR_INTERNAL: return "internal error";
    default: return "unknown status";
  }
}

const char* tc_last_error(void) { return t_last_error.c_str(); }

tc_status tc_batch_from_ijk(const int32_t* d_ijk, const int64_t* h_offsets, int32_t grid_count,
                            const tc_allocator* allocator, void* stream, tc_grid_batch** out) {
  if (!out) return fail(TC_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (grid_count < 1) return fail(TC_ERR_INVALID_ARG, "grid_count must be >= 1");
  if (!h_offsets) return fail(TC_ERR_INVALID_ARG, "h_offsets is NULL");
  if (h_offsets[0] != 0) return fail(TC_ERR_INVALID_ARG, "h_offsets[0] must be 0");
  for (int32_t g = 0; g < grid_count; ++g)
    if (h_offsets[g + 1] < h_offsets[g]) return fail(TC_ERR_INVALID_ARG, "h_offsets must be non-decreasing");
  const int64_t n = h_offsets[grid_count];
  if (n >= (1ll << 30)) return fail(TC_ERR_UNSUPPORTED, "more than 2^30 voxel rows");
  if (n > 0 && !d_ijk) return fail(TC_ERR_INVALID_ARG, "d_ijk is NULL");
  if (allocator && (!allocator->alloc || !allocator->free))
    return fail(TC_ERR_INVALID_ARG, "allocator callbacks are NULL");
  return guarded([&]() {
    tc::SourceScope scope(allocator);
    *out = tc::finish_batch(
        tc::build_from_ijk(d_ijk, h_offsets, grid_count, tc::OutAlloc{allocator, (hipStream_t)stream}),
        (hipStream_t)stream);
    return TC_OK;
  });
}

tc_status tc_batch_from_points(const float* d_xyz, const int64_t* h_offsets, int32_t grid_count,
                              const float* h_voxel_size, const float* h_origin, int32_t mode,
                              const tc_allocator* allocator, void* stream, tc_grid_batch** out) {
  if (!out) return fail(TC_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (grid_count < 1) return fail(TC_ERR_INVALID_ARG, "grid_count must be >= 1");
  if (!h_offsets || !h_voxel_size || !h_origin) return fail(TC_ERR_INVALID_ARG, "NULL host argument");
  if (mode != 0 && mode != 1) return fail(TC_ERR_INVALID_ARG, "mode must be 0 or 1");
  if (h_offsets[0] != 0) return fail(TC_ERR_INVALID_ARG, "h_offsets[0] must be 0");
  for (int32_t g = 0; g < grid_count; ++g) {
    if (h_offsets[g + 1] < h_offsets[g]) return fail(TC_ERR_INVALID_ARG, "h_offsets must be non-decreasing");
    for (int k = 0; k < 3; ++k) {
      const float vs = h_voxel_size[g * 3 + k], o = h_origin[g * 3 + k];
      if (!std::isfinite(vs) || !(vs > 0.0f)) return fail(TC_ERR_INVALID_ARG, "voxel sizes must be finite and > 0");
      if (!std::isfinite(o)) return fail(TC_ERR_INVALID_ARG, "origins must be finite");
    }
  }
  const int64_t n = h_offsets[grid_count];
  if ((mode == 0 ? n : 8 * n) >= (1ll << 30)) return fail(TC_ERR_UNSUPPORTED, "more than 2^30 voxel rows");
  if (n > 0 && !d_xyz) return fail(TC_ERR_INVALID_ARG, "d_xyz is NULL");
  if (allocator && (!allocator->alloc || !allocator->free))
    return fail(TC_ERR_INVALID_ARG, "allocator callbacks are NULL");
  return guarded([&]() {
    tc::SourceScope scope(allocator);
    *out = tc::finish_batch(tc::build_from_points(d_xyz, h_offsets, grid_count, h_voxel_size, h_origin, mode,
                                                  tc::OutAlloc{allocator, (hipStream_t)stream}),
                            (hipStream_t)stream);
    return TC_OK;
  });
}

tc_status tc_build_batched_topology(const tc_grid_batch* src, int32_t op, int32_t factor,
                                    const tc_allocator* allocator, void* stream, tc_grid_batch** out) {
  return tc_build_batched_topology_many(src, 1, &op, &factor, allocator, stream, out);
}

tc_status tc_build_batched_topology_many(const tc_grid_batch* src, int32_t n_ops, const int32_t* h_ops,
                                         const int32_t* h_factors, const tc_allocator* allocator, void* stream,
                                         tc_grid_batch** out) {
  if (!out) return fail(TC_ERR_INVALID_ARG, "out is NULL");
  if (n_ops < 1) return fail(TC_ERR_INVALID_ARG, "n_ops must be >= 1");
  for (int32_t i = 0; i < n_ops; ++i) out[i] = nullptr;
  if (!h_ops || !h_factors) return fail(TC_ERR_INVALID_ARG, "h_ops or h_factors is NULL");
  if (!src) return fail(TC_ERR_INVALID_ARG, "src is NULL");
  if (allocator && (!allocator->alloc || !allocator->free))
    return fail(TC_ERR_INVALID_ARG, "allocator callbacks are NULL");
  std::vector<std::vector<int>> plan(n_ops);
  for (int32_t i = 0; i < n_ops; ++i) {
    std::string msg;
    const tc_status st = tc::op_passes(h_ops[i], h_factors[i], plan[i], msg);
    if (st != TC_OK) return fail(st, n_ops > 1 ? "op " + std::to_string(i) + ": " + msg : msg);
  }
  std::vector<tc_grid_batch*> made(n_ops, nullptr);
  const tc_status st = guarded([&]() {
    if (current_device() != src->device) throw tc::Error(TC_ERR_INVALID_ARG, "src lives on another device");
    tc::SourceScope scope(allocator);
    hipStream_t s = (hipStream_t)stream;
    if (n_ops == 1) {  // one target: its passes on the caller's stream, each waiting for its own counts
      const std::vector<int>& passes = plan[0];
      if (passes.empty()) {  // kernel size 1: the target is the source
        made[0] = tc::copy_batch(src, tc::OutAlloc{allocator, s});
      } else {
        const tc_grid_batch* cur = src;
        tc_grid_batch* owned = nullptr;  // intermediate result of the previous pass
        try {
          for (size_t p = 0; p < passes.size(); ++p) {
            const bool last = p + 1 == passes.size();
            tc_grid_batch* next = tc::build_pass(cur, passes[p], tc::OutAlloc{allocator, s, !last});
            tc::free_batch(owned);
            owned = next;
            cur = next;
          }
        } catch (...) {
          tc::free_batch(owned);
          throw;
        }
        made[0] = owned;
      }
    } else {
      // Several targets, longest chain first: the first runs on s, the others on
      // kSideStreams internal streams (round robin) that wait once for all earlier
      // work on s, so that the targets' kernel chains overlap on the device. The
      // passes go out round by round (every target's first pass, then the second
      // passes, ...), each leaving its header readback pending, so that a chain's
      // next pass finds the counts of its intermediate ready when it starts.
      // Outputs are allocated on s. An output whose pass left its headers pending
      // is complete once they are read (its finalize is its last kernel); for any
      // other output built on an internal stream (a large batch's writers, a
      // copy) s waits for that stream before the call returns, so later work on s,
      // and reuse of its memory in s order, comes after the kernels that wrote it.
      // Cross-stream waits cost the host several microseconds each, hence one
      // side stream and no join when nothing needs it.
      const int dev = src->device;
      const int nside = std::min<int>(n_ops - 1, tc::kSideStreams);
      std::vector<int32_t> order(n_ops);
      for (int32_t i = 0; i < n_ops; ++i) order[i] = i;
      std::stable_sort(order.begin(), order.end(),
                       [&](int32_t a, int32_t b) { return plan[a].size() > plan[b].size(); });
      std::vector<hipEvent_t> evs;
      auto ev_take = [&]() {
        evs.push_back(tc::pending_event_take(dev));
        return evs.back();
      };
      auto give_events = [&]() {
        for (hipEvent_t e : evs) tc::pending_event_give(dev, e);
        evs.clear();
      };
      std::vector<char> needs_join(nside, 0);
      auto join = [&](bool all) {  // s waits for the side streams that need it
        for (int k = 0; k < nside; ++k) {
          if (!all && !needs_join[k]) continue;
          needs_join[k] = 0;
          hipEvent_t e = ev_take();
          tc::hip_check(hipEventRecord(e, tc::internal_stream(dev, k)), "hipEventRecord");
          tc::hip_check(hipStreamWaitEvent(s, e, 0), "hipStreamWaitEvent");
        }
      };
      std::vector<const tc_grid_batch*> cur(n_ops, src);
      std::vector<tc_grid_batch*> owned(n_ops, nullptr);  // intermediates of chains
      bool started = false;
      try {
        if (nside > 0) {
          hipEvent_t e0 = ev_take();
          tc::hip_check(hipEventRecord(e0, s), "hipEventRecord");
          for (int k = 0; k < nside; ++k)
            tc::hip_check(hipStreamWaitEvent(tc::internal_stream(dev, k), e0, 0), "hipStreamWaitEvent");
        }
        started = true;
        const size_t rounds = std::max<size_t>(1, plan[order[0]].size());
        for (size_t r = 0; r < rounds; ++r) {
          for (int32_t q = 0; q < n_ops; ++q) {
            const int32_t i = order[q];
            const int side = q == 0 ? -1 : (q - 1) % nside;
            const hipStream_t si = side < 0 ? s : tc::internal_stream(dev, side);
            const std::vector<int>& passes = plan[i];
            if (passes.empty()) {  // kernel size 1: a copy of the source
              if (r == 0) {
                made[i] = tc::copy_batch(src, tc::OutAlloc{allocator, si, false, s});
                if (side >= 0) needs_join[side] = 1;
              }
              continue;
            }
            if (r >= passes.size()) continue;
            const bool last = r + 1 == passes.size();
            tc_grid_batch* next = tc::build_pass(
                cur[i], passes[r], tc::OutAlloc{allocator, si, !last, last && side >= 0 ? s : nullptr}, nullptr, true);
            if (last && side >= 0 && !next->hdr_pending) needs_join[side] = 1;
            tc::free_batch(owned[i]);  // its readers are on si, before any later reuse on si
            owned[i] = last ? nullptr : next;
            cur[i] = next;
            if (last) made[i] = next;
          }
        }
        join(false);
      } catch (...) {
        if (started) {
          try {
            join(true);
          } catch (...) {
          }
        }
        for (int32_t i = 0; i < n_ops; ++i) tc::free_batch(owned[i]);
        give_events();
        throw;
      }
      give_events();
    }
    for (int32_t i = 0; i < n_ops; ++i) tc::resolve_counts(made[i]);
    for (int32_t i = 0; i < n_ops; ++i) {
      tc::queue_voxel_total(made[i], s);  // no-op where the headers gave the total
      out[i] = made[i];
    }
    return TC_OK;
  });
  if (st != TC_OK) {
    for (int32_t i = 0; i < n_ops; ++i) {
      tc::free_batch(made[i]);
      out[i] = nullptr;
    }
  }
  return st;
}

tc_status tc_build_masked_refine(const tc_grid_batch* src, const uint8_t* d_keep, int64_t n_keep, int32_t factor,
                                 const tc_allocator* allocator, void* stream, tc_grid_batch** out) {
  if (!out) return fail(TC_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!src) return fail(TC_ERR_INVALID_ARG, "src is NULL");
  if (allocator && (!allocator->alloc || !allocator->free))
    return fail(TC_ERR_INVALID_ARG, "allocator callbacks are NULL");
  if (factor != 2 && factor != 4 && factor != 8)
    return fail(factor < 2 ? TC_ERR_INVALID_ARG : TC_ERR_UNSUPPORTED, "refine factor must be 2, 4 or 8");
  return guarded([&]() {
    if (current_device() != src->device) throw tc::Error(TC_ERR_INVALID_ARG, "src lives on another device");
    tc::SourceScope scope(allocator);
    hipStream_t s = (hipStream_t)stream;
    const int64_t total = tc::read_voxel_total(src, s);
    if (n_keep != total)
      throw tc::Error(TC_ERR_INVALID_ARG, "keep holds " + std::to_string(n_keep) + " flags for " +
                                              std::to_string(total) + " voxels");
    if (total > 0 && !d_keep) throw tc::Error(TC_ERR_INVALID_ARG, "d_keep is NULL");
    // masked copies of the source leaf masks (plus a consistency flag), then the
    // refine passes; the first reads the masked copies
    tc::Arena a(s);
    const size_t o_mask = a.reserve(64 * (size_t)src->nl);
    const size_t o_flag = a.reserve(4);
    a.commit();
    tc::u64* masked = a.at<tc::u64>(o_mask);
    int32_t* flag = a.at<int32_t>(o_flag);
    tc::fill_i32(flag, 0, 1, nullptr, 1, s);
    tc::mask_leaves(src, d_keep, n_keep, masked, flag, s);
    const int npass = factor == 2 ? 1 : (factor == 4 ? 2 : 3);
    const tc_grid_batch* cur = src;
    tc_grid_batch* owned = nullptr;
    try {
      for (int p = 0; p < npass; ++p) {
        const bool last = p + 1 == npass;
        tc_grid_batch* next = tc::build_pass(cur, TC_OP_REFINE, tc::OutAlloc{allocator, s, !last},
                                             p == 0 ? masked : nullptr);
        if (p == 0) {
          int32_t* h = static_cast<int32_t*>(tc::pinned_staging(64));
          tc::hip_check(hipMemcpyAsync(h, flag, 4, hipMemcpyDeviceToHost, s), "readback");
          tc::hip_check(hipStreamSynchronize(s), "hipStreamSynchronize");
          if (h[0] != 0) {
            tc::free_batch(next);
            throw tc::Error(TC_ERR_INTERNAL, "masked refine: keep index out of range");
          }
        }
        tc::free_batch(owned);
        owned = next;
        cur = next;
      }
    } catch (...) {
      tc::free_batch(owned);
      throw;
    }
    *out = tc::finish_batch(owned, s);
    return TC_OK;
  });
}

tc_status tc_batch_get_info(const tc_grid_batch* b, tc_batch_info* out) {
  if (!b || !out) return fail(TC_ERR_INVALID_ARG, "NULL argument");
  const tc::GridView v = b->view();
  out->grid_count = b->B;
  out->upper_count = b->n2;
  out->lower_count = b->n1;
  out->leaf_count = b->nl;
  out->h_upper_counts = b->h_upper.data();
  out->h_lower_counts = b->h_lower.data();
  out->h_leaf_counts = b->h_leaf.data();
  out->d_buffer = b->buffer;
  out->buffer_bytes = b->bytes;
  out->d_headers = v.headers;
  out->d_upper_origin = reinterpret_cast<const int32_t*>(v.upper_origin);
  out->d_upper_key = v.upper_key;
  out->d_upper_first = v.upper_first;
  out->d_upper_mask = v.upper_mask;
  out->d_lower_origin = reinterpret_cast<const int32_t*>(v.lower_origin);
  out->d_lower_first = v.lower_first;
  out->d_lower_mask = v.lower_mask;
  out->d_lower_prefix = v.lower_prefix;
  out->d_leaf_origin = reinterpret_cast<const int32_t*>(v.leaf_origin);
  out->d_leaf_parent = v.leaf_parent;
  out->d_leaf_mask = v.leaf_mask;
  out->d_leaf_prefix = v.leaf_prefix;
  out->d_leaf_offset = v.leaf_offset;
  return TC_OK;
}

tc_status tc_batch_read_headers(const tc_grid_batch* b, tc_grid_header* h_out, void* stream) {
  if (!b || !h_out) return fail(TC_ERR_INVALID_ARG, "NULL argument");
  return guarded([&]() {
    tc::read_voxel_total(b, (hipStream_t)stream);  // the status check; usually no extra wait
    const size_t bytes = sizeof(tc_grid_header) * (size_t)b->B;
    void* h = tc::pinned_staging(bytes);
    hipStream_t s = (hipStream_t)stream;
    tc::hip_check(hipMemcpyAsync(h, b->view().headers, bytes, hipMemcpyDeviceToHost, s), "header readback");
    tc::hip_check(hipStreamSynchronize(s), "hipStreamSynchronize");
    std::memcpy(h_out, h, bytes);
    const tc_grid_header& last = h_out[b->B - 1];
    b->vox_total = last.voxel_begin + last.voxel_count;
    b->vox_known = true;
    return TC_OK;
  });
}

tc_status tc_batch_voxel_total(const tc_grid_batch* b, int64_t* h_total, void* stream) {
  if (!b || !h_total) return fail(TC_ERR_INVALID_ARG, "NULL argument");
  return guarded([&]() {
    *h_total = tc::read_voxel_total(b, (hipStream_t)stream);
    return TC_OK;
  });
}

tc_status tc_enumerate_ijk(const tc_grid_batch* b, int32_t* d_ijk_out, int64_t capacity, void* stream) {
  if (!b) return fail(TC_ERR_INVALID_ARG, "batch is NULL");
  return guarded([&]() {
    hipStream_t s = (hipStream_t)stream;
    const int64_t total = tc::read_voxel_total(b, s);
    if (total == 0) return TC_OK;
    if (!d_ijk_out) throw tc::Error(TC_ERR_INVALID_ARG, "d_ijk_out is NULL");
    if (capacity < total)
      throw tc::Error(TC_ERR_INVALID_ARG, "capacity " + std::to_string(capacity) + " < voxel total " +
                                              std::to_string(total));
    tc::tree_enumerate(b->view(), d_ijk_out, s);
    return TC_OK;
  });
}

tc_status tc_enumerate_ijk_many(int32_t n, const tc_grid_batch* const* batches, int32_t* const* d_ijk_outs,
                                const int64_t* capacities, void* stream) {
  if (n < 1) return fail(TC_ERR_INVALID_ARG, "n must be >= 1");
  if (!batches || !d_ijk_outs || !capacities) return fail(TC_ERR_INVALID_ARG, "NULL argument");
  for (int32_t j = 0; j < n; ++j)
    if (!batches[j]) return fail(TC_ERR_INVALID_ARG, "batch " + std::to_string(j) + " is NULL");
  return guarded([&]() {
    hipStream_t s = (hipStream_t)stream;
    const int dev = current_device();
    std::vector<tc::GridView> views;
    std::vector<int32_t*> outs;
    views.reserve(n);
    outs.reserve(n);
    for (int32_t j = 0; j < n; ++j) {
      const tc_grid_batch* b = batches[j];
      if (b->device != dev) throw tc::Error(TC_ERR_INVALID_ARG, "batch " + std::to_string(j) + " lives on another device");
      const int64_t total = tc::read_voxel_total(b, s);
      if (total == 0) continue;
      if (!d_ijk_outs[j]) throw tc::Error(TC_ERR_INVALID_ARG, "d_ijk_outs[" + std::to_string(j) + "] is NULL");
      if (capacities[j] < total)
        throw tc::Error(TC_ERR_INVALID_ARG, "capacity " + std::to_string(capacities[j]) + " < voxel total " +
                                                std::to_string(total) + " of batch " + std::to_string(j));
      views.push_back(b->view());
      outs.push_back(d_ijk_outs[j]);
    }
    if (!views.empty()) tc::tree_enumerate_many(views.data(), outs.data(), (int)views.size(), s);
    return TC_OK;
  });
}

tc_status tc_build_kernel_map(const tc_grid_batch* src, const tc_grid_batch* dst, int32_t kernel_size,
                              int32_t stride, int32_t transposed, int32_t* d_out, int64_t capacity,
                              void* stream) {
  if (!src || !dst) return fail(TC_ERR_INVALID_ARG, "batch is NULL");
  if (src->B != dst->B) return fail(TC_ERR_INVALID_ARG, "source and target member counts differ");
  if (kernel_size < 1 || kernel_size > 8) return fail(TC_ERR_INVALID_ARG, "kernel_size must be in [1, 8]");
  if (stride < 1) return fail(TC_ERR_INVALID_ARG, "stride must be positive");
  if (stride > 2) return fail(TC_ERR_UNSUPPORTED, "stride must be 1 or 2");
  if (transposed != 0 && transposed != 1) return fail(TC_ERR_INVALID_ARG, "transposed must be 0 or 1");
  return guarded([&]() {
    hipStream_t s = (hipStream_t)stream;
    const int64_t n_src = tc::read_voxel_total(src, s);
    if (n_src > (int64_t)INT32_MAX) throw tc::Error(TC_ERR_UNSUPPORTED, "source voxel indices exceed int32");
    const int64_t kk = (int64_t)kernel_size * kernel_size * kernel_size;
    const int64_t need = tc::read_voxel_total(dst, s) * kk;
    if (need == 0) return TC_OK;
    if (!d_out) throw tc::Error(TC_ERR_INVALID_ARG, "d_out is NULL");
    if (capacity < need)
      throw tc::Error(TC_ERR_INVALID_ARG,
                      "capacity " + std::to_string(capacity) + " < " + std::to_string(need) + " entries");
    tc::kernel_map(src->view(), dst->view(), kernel_size, stride, transposed, d_out, need, s);
    return TC_OK;
  });
}

tc_status tc_build_kernel_map_noalloc(const tc_grid_batch* src, const tc_grid_batch* dst, int32_t kernel_size,
                                      int32_t stride, int32_t transposed, int32_t* d_out, int64_t capacity,
                                      void* stream) {
  if (!src || !dst) return fail(TC_ERR_INVALID_ARG, "batch is NULL");
  if (src->B != dst->B) return fail(TC_ERR_INVALID_ARG, "source and target member counts differ");
  if (kernel_size < 1 || kernel_size > 8) return fail(TC_ERR_INVALID_ARG, "kernel_size must be in [1, 8]");
  if (stride < 1) return fail(TC_ERR_INVALID_ARG, "stride must be positive");
  if (stride > 2) return fail(TC_ERR_UNSUPPORTED, "stride must be 1 or 2");
  if (transposed != 0 && transposed != 1) return fail(TC_ERR_INVALID_ARG, "transposed must be 0 or 1");
  return guarded([&]() {
    if (current_device() != src->device || current_device() != dst->device)
      throw tc::Error(TC_ERR_INVALID_ARG, "a batch lives on another device");
    hipStream_t s = (hipStream_t)stream;
    size_t cap = 0;
    char* scratch = tc::noalloc_scratch(&cap);  // set-up on the first call on this device
    const int64_t n_src = tc::read_voxel_total(src, s, true);
    if (n_src > (int64_t)INT32_MAX) throw tc::Error(TC_ERR_UNSUPPORTED, "source voxel indices exceed int32");
    const int64_t kk = (int64_t)kernel_size * kernel_size * kernel_size;
    const int64_t need = tc::read_voxel_total(dst, s, true) * kk;
    if (need == 0) return TC_OK;
    if (!d_out) throw tc::Error(TC_ERR_INVALID_ARG, "d_out is NULL");
    if (capacity < need)
      throw tc::Error(TC_ERR_INVALID_ARG,
                      "capacity " + std::to_string(capacity) + " < " + std::to_string(need) + " entries");
    const size_t want = tc::kernel_map_scratch_bytes(src->view(), dst->view(), kernel_size, stride, transposed);
    if (want > cap)
      throw tc::Error(TC_ERR_UNSUPPORTED, "kernel map needs " + std::to_string(want) +
                                              " bytes of scratch; the no-allocation entry point has " +
                                              std::to_string(cap) + " (use tc_build_kernel_map)");
    tc::kernel_map(src->view(), dst->view(), kernel_size, stride, transposed, d_out, need, s, scratch, cap);
    return TC_OK;
  });
}

tc_status tc_scratch_release(void) {
  return guarded([&]() {
    tc::scratch_release_all();
    tc::batch_buffers_release();
    return TC_OK;
  });
}

void tc_batch_free(tc_grid_batch* b) {
  try {
    tc::free_batch(b);
  } catch (...) {
  }
}

tc_status tc_debug_inject_flags(int32_t bits) {
  if (bits < 0 || bits > 3) return fail(TC_ERR_INVALID_ARG, "bits must be in [0, 3]");
  tc::debug_set_inject(bits);
  return TC_OK;
}

tc_status tc_debug_wide_loads(int32_t on) {
  if (on != 0 && on != 1) return fail(TC_ERR_INVALID_ARG, "on must be 0 or 1");
  tc::debug_set_wide_loads(on == 1);
  return TC_OK;
}

tc_status tc_profile_enable(const char* kernel_names) {
  if (!kernel_names) return fail(TC_ERR_INVALID_ARG, "kernel_names is NULL");
  return guarded([&]() {
    tc::prof_enable(kernel_names);
    return TC_OK;
  });
}

tc_status tc_profile_read(const char* kernel_name, double* h_total_ms, int64_t* h_launches) {
  if (!kernel_name || !h_total_ms || !h_launches) return fail(TC_ERR_INVALID_ARG, "NULL argument");
  return guarded([&]() {
    tc::prof_read(kernel_name, h_total_ms, h_launches);
    return TC_OK;
  });
}

tc_status tc_profile_disable(void) {
  return guarded([&]() {
    tc::prof_disable();
    return TC_OK;
  });
}

}  // extern "C"
