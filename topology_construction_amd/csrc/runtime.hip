// Host runtime helpers: stream-ordered scratch memory, pinned staging buffers,
// kernel timing with HIP events.
#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "internal.hpp"

namespace tc {

// ------------------------------------------------------------------ device memory
static std::mutex g_pool_mu;
static std::vector<int> g_pool_ready;

static void ensure_pool(int dev) {
  std::lock_guard<std::mutex> lk(g_pool_mu);
  if ((int)g_pool_ready.size() <= dev) g_pool_ready.resize(dev + 1, 0);
  if (g_pool_ready[dev]) return;
  hipMemPool_t pool;
  hip_check(hipDeviceGetDefaultMemPool(&pool, dev), "hipDeviceGetDefaultMemPool");
  uint64_t threshold = ~0ull;  // keep freed blocks cached in the pool
  hip_check(hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &threshold),
            "hipMemPoolSetAttribute");
  g_pool_ready[dev] = 1;
}

void* device_alloc_async(size_t bytes, hipStream_t s) {
  int dev = 0;
  hip_check(hipGetDevice(&dev), "hipGetDevice");
  ensure_pool(dev);
  void* p = nullptr;
  hipError_t e = hipMallocAsync(&p, bytes ? bytes : 256, s);
  if (e == hipErrorOutOfMemory || (e == hipSuccess && !p)) {
    (void)hipGetLastError();
    throw Error(TC_ERR_ALLOC, "hipMallocAsync: out of device memory (" + std::to_string(bytes) + " bytes)");
  }
  hip_check(e, "hipMallocAsync");
  return p;
}

void device_free_async(void* p, hipStream_t s) {
  if (p) (void)hipFreeAsync(p, s);
}

// ------------------------------------------------------------------ memory sources
// The device memory of a call (scratch arenas, intermediate batches of chained
// passes) comes from the allocator its entry point was given, or from the
// device's stream-ordered pool when it was given none. The entry point names
// the source for its thread with a SourceScope.
namespace {
thread_local tc_allocator t_src{};
thread_local bool t_src_set = false;

bool same_source(const tc_allocator& a, bool a_set, const tc_allocator& b, bool b_set) {
  if (a_set != b_set) return false;
  return !a_set || (a.alloc == b.alloc && a.free == b.free && a.ctx == b.ctx);
}
}  // namespace

SourceScope::SourceScope(const tc_allocator* a) : prev_(t_src), prev_set_(t_src_set) {
  t_src_set = a != nullptr;
  t_src = a ? *a : tc_allocator{};
}
SourceScope::~SourceScope() {
  t_src = prev_;
  t_src_set = prev_set_;
}

// ------------------------------------------------------------------ scratch cache
// Process-wide cache of scratch blocks keyed by (device, stream, source). An
// arena takes the smallest idle block of its key that fits, else replaces the
// largest idle block of its key (or adds one), and marks it busy until it is
// given back; nothing is freed on the per-call path, and reuse is ordered by
// the stream itself. Idle blocks beyond kIdleBlocks, or beyond kIdleBytes in
// total, are freed oldest first (after a device synchronisation when they
// belong to another stream, which may since have been destroyed).
struct ScratchBlock {
  int device;
  hipStream_t stream;
  tc_allocator src;
  bool src_set;
  char* p;
  size_t bytes;
  bool busy;
  uint64_t stamp;
};

namespace {
constexpr size_t kIdleBlocks = 24;
constexpr size_t kIdleBytes = size_t(8) << 30;

struct ScratchCache {
  std::mutex mu;
  std::vector<ScratchBlock*> blocks;  // stable addresses: arenas hold the pointer
  uint64_t clock = 0;
};
ScratchCache& scratch_cache() {
  static ScratchCache* c = new ScratchCache();  // never destroyed: no frees during process teardown
  return *c;
}

char* source_alloc(const tc_allocator& src, bool src_set, size_t bytes, hipStream_t s) {
  if (!src_set) return static_cast<char*>(device_alloc_async(bytes, s));
  void* p = src.alloc(src.ctx, bytes, (void*)s);
  if (!p) throw Error(TC_ERR_ALLOC, "allocator returned NULL for " + std::to_string(bytes) + " bytes of scratch");
  return static_cast<char*>(p);
}

// Frees a block that no queued work uses any more on `s` (its own stream) or
// anywhere (synced = true after a device synchronisation).
void block_free(ScratchBlock* b, hipStream_t s, bool synced) {
  if (!b->p) return;
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return;
  if (b->device != cur && hipSetDevice(b->device) != hipSuccess) return;
  if (b->src_set) {
    b->src.free(b->src.ctx, b->p, b->bytes, (void*)b->stream);
  } else {
    device_free_async(b->p, synced ? nullptr : s);
  }
  if (b->device != cur) (void)hipSetDevice(cur);
  b->p = nullptr;
  b->bytes = 0;
}

// Drops idle blocks beyond the cache limits (caller holds no lock).
void scratch_trim(hipStream_t s) {
  ScratchCache& c = scratch_cache();
  std::vector<ScratchBlock*> drop;
  {
    std::lock_guard<std::mutex> lk(c.mu);
    for (;;) {
      size_t idle = 0, idle_bytes = 0;
      ScratchBlock* oldest = nullptr;
      for (ScratchBlock* b : c.blocks)
        if (!b->busy) {
          ++idle;
          idle_bytes += b->bytes;
          if (!oldest || b->stamp < oldest->stamp) oldest = b;
        }
      if (!oldest || (idle <= kIdleBlocks && idle_bytes <= kIdleBytes)) break;
      c.blocks.erase(std::find(c.blocks.begin(), c.blocks.end(), oldest));
      drop.push_back(oldest);
    }
  }
  bool synced = false;
  for (ScratchBlock* b : drop) {
    if (b->stream != s && !synced) synced = hipDeviceSynchronize() == hipSuccess;
    block_free(b, s, b->stream != s);
    delete b;
  }
}
}  // namespace

ScratchBlock* scratch_acquire(size_t bytes, hipStream_t s) {
  int dev = 0;
  hip_check(hipGetDevice(&dev), "hipGetDevice");
  ScratchCache& c = scratch_cache();
  ScratchBlock* fit = nullptr;
  ScratchBlock* victim = nullptr;
  {
    std::lock_guard<std::mutex> lk(c.mu);
    for (ScratchBlock* b : c.blocks) {
      if (b->busy || b->device != dev || b->stream != s || !same_source(b->src, b->src_set, t_src, t_src_set))
        continue;
      if (b->bytes >= bytes && (!fit || b->bytes < fit->bytes)) fit = b;
      if (!victim || b->bytes > victim->bytes) victim = b;
    }
    if (fit) {
      fit->busy = true;
      fit->stamp = ++c.clock;
      return fit;
    }
    if (victim) victim->busy = true;  // replaced below, outside the lock (callbacks may be slow)
  }
  // grow: a new block a quarter larger than asked, in place of the largest idle one
  const size_t want = bytes + bytes / 4 + 4096;
  if (victim) block_free(victim, s, false);
  char* p = nullptr;
  try {
    p = source_alloc(t_src, t_src_set, want, s);
  } catch (...) {
    if (victim) {
      std::lock_guard<std::mutex> lk(c.mu);
      c.blocks.erase(std::find(c.blocks.begin(), c.blocks.end(), victim));
      delete victim;
    }
    throw;
  }
  std::lock_guard<std::mutex> lk(c.mu);
  ScratchBlock* b = victim;
  if (!b) {
    b = new ScratchBlock();
    c.blocks.push_back(b);
  }
  *b = ScratchBlock{dev, s, t_src, t_src_set, p, want, true, ++c.clock};
  return b;
}

void scratch_give_back(ScratchBlock* b, hipStream_t s) {
  if (!b) return;
  {
    ScratchCache& c = scratch_cache();
    std::lock_guard<std::mutex> lk(c.mu);
    b->busy = false;
    b->stamp = ++c.clock;
  }
  scratch_trim(s);
}

char* scratch_ptr(const ScratchBlock* b) { return b ? b->p : nullptr; }

void scratch_release_all() {
  ScratchCache& c = scratch_cache();
  std::vector<ScratchBlock*> drop;
  {
    std::lock_guard<std::mutex> lk(c.mu);
    std::vector<ScratchBlock*> keep;
    for (ScratchBlock* b : c.blocks) (b->busy ? keep : drop).push_back(b);
    c.blocks.swap(keep);
  }
  if (drop.empty()) return;
  hip_check(hipDeviceSynchronize(), "hipDeviceSynchronize");
  for (ScratchBlock* b : drop) {
    block_free(b, nullptr, true);
    delete b;
  }
}

size_t scratch_cached_bytes() {
  ScratchCache& c = scratch_cache();
  std::lock_guard<std::mutex> lk(c.mu);
  size_t n = 0;
  for (const ScratchBlock* b : c.blocks) n += b->bytes;
  return n;
}

// ------------------------------------------------------------------ batch buffers
// Buffers of batches built without an allocator: tc_batch_free hands them back
// here, and the next batch on the same device and stream that fits (using at
// least half of the buffer) takes one instead of allocating. Reuse is ordered
// by that stream, as a stream-ordered free would be.
namespace {
struct CachedBuffer {
  int device;
  hipStream_t stream;
  void* p;
  size_t cap;
};
std::mutex g_buf_mu;
std::vector<CachedBuffer> g_bufs;
size_t g_buf_bytes = 0;
constexpr size_t kBufCacheBytes = size_t(4) << 30;  // beyond this the oldest buffers are freed
constexpr size_t kBufCacheCount = 64;
}  // namespace

void* batch_buffer_take(size_t bytes, hipStream_t s, size_t* cap) {
  int dev = 0;
  hip_check(hipGetDevice(&dev), "hipGetDevice");
  {
    std::lock_guard<std::mutex> lk(g_buf_mu);
    int best = -1;
    for (int i = 0; i < (int)g_bufs.size(); ++i) {
      const CachedBuffer& c = g_bufs[i];
      if (c.device != dev || c.stream != s || c.cap < bytes || c.cap / 2 > bytes) continue;
      if (best < 0 || c.cap < g_bufs[best].cap) best = i;
    }
    if (best >= 0) {
      void* p = g_bufs[best].p;
      *cap = g_bufs[best].cap;
      g_buf_bytes -= g_bufs[best].cap;
      g_bufs.erase(g_bufs.begin() + best);
      return p;
    }
  }
  *cap = bytes ? bytes : 256;
  return device_alloc_async(*cap, s);
}

void batch_buffer_give(void* p, size_t cap, int device, hipStream_t s) {
  if (!p) return;
  std::vector<CachedBuffer> drop;
  {
    std::lock_guard<std::mutex> lk(g_buf_mu);
    g_bufs.push_back(CachedBuffer{device, s, p, cap});
    g_buf_bytes += cap;
    while (!g_bufs.empty() && (g_buf_bytes > kBufCacheBytes || g_bufs.size() > kBufCacheCount)) {
      drop.push_back(g_bufs.front());
      g_buf_bytes -= g_bufs.front().cap;
      g_bufs.erase(g_bufs.begin());
    }
  }
  for (const CachedBuffer& c : drop) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) continue;
    if (c.device != cur) (void)hipSetDevice(c.device);
    device_free_async(c.p, c.stream);
    if (c.device != cur) (void)hipSetDevice(cur);
  }
}

void batch_buffers_release() {
  std::vector<CachedBuffer> drop;
  {
    std::lock_guard<std::mutex> lk(g_buf_mu);
    drop.swap(g_bufs);
    g_buf_bytes = 0;
  }
  int cur = 0;
  hip_check(hipGetDevice(&cur), "hipGetDevice");
  for (const CachedBuffer& c : drop) {
    if (c.device != cur) hip_check(hipSetDevice(c.device), "hipSetDevice");
    device_free_async(c.p, c.stream);
    if (c.device != cur) hip_check(hipSetDevice(cur), "hipSetDevice");
  }
}

void Arena::commit() {
  if (base_) throw Error(TC_ERR_INTERNAL, "arena committed twice");
  block_ = scratch_acquire(size_, stream_);
  base_ = scratch_ptr(block_);
}

void Arena::release() {
  if (block_) scratch_give_back(block_, stream_);
  base_ = nullptr;
  block_ = nullptr;
}

// ------------------------------------------------------------------ pinned staging
namespace {
struct Pinned {
  void* p = nullptr;
  size_t bytes = 0;
};
thread_local Pinned t_pinned;
}  // namespace

void* pinned_staging(size_t bytes) {
  if (t_pinned.bytes >= bytes && t_pinned.p) return t_pinned.p;
  size_t want = 4096;
  while (want < bytes) want <<= 1;
  if (t_pinned.p) (void)hipHostFree(t_pinned.p);
  t_pinned.p = nullptr;
  t_pinned.bytes = 0;
  void* p = nullptr;
  hip_check(hipHostMalloc(&p, want, hipHostMallocDefault), "hipHostMalloc");
  t_pinned.p = p;
  t_pinned.bytes = want;
  return p;
}

// ------------------------------------------------------------------ device facts
int device_cu_count() {
  static int cached[64];  // 0 = not read yet (a benign race: every reader stores the same value)
  int dev = 0;
  hip_check(hipGetDevice(&dev), "hipGetDevice");
  if (dev >= 0 && dev < 64 && cached[dev] > 0) return cached[dev];
  int cus = 0;
  hip_check(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev), "hipDeviceGetAttribute");
  if (cus <= 0) cus = 1;
  if (dev >= 0 && dev < 64) cached[dev] = cus;
  return cus;
}

// ------------------------------------------------------------------ voxel-total slots
namespace {
constexpr int kVoxChunk = 256;  // slots per pinned allocation, 64 bytes each
struct VoxSlot {
  int64_t* h;
  hipEvent_t ev;
  int device;
};
struct VoxPool {
  std::mutex mu;
  std::vector<VoxSlot> slots;
  std::vector<int> idle;
};
VoxPool& vox_pool() {
  static VoxPool* p = new VoxPool();  // never destroyed: batches may outlive static teardown
  return *p;
}
}  // namespace

// ------------------------------------------------------------------ pending headers
// Pinned host blocks (power-of-two sizes, from 4 KiB) and timing-free events
// per device, kept between uses: a batch whose headers are still on their way
// holds one of each until its counts are resolved.
namespace {
struct PendingPool {
  std::mutex mu;
  std::vector<std::pair<void*, size_t>> blocks;
  std::vector<std::pair<int, hipEvent_t>> events;
};
PendingPool& pending_pool() {
  static PendingPool* p = new PendingPool();  // never destroyed: batches may outlive static teardown
  return *p;
}
}  // namespace

void* pinned_block_take(size_t bytes, size_t* cap) {
  size_t want = 4096;
  while (want < bytes) want <<= 1;
  PendingPool& pp = pending_pool();
  {
    std::lock_guard<std::mutex> lk(pp.mu);
    for (size_t k = 0; k < pp.blocks.size(); ++k) {
      if (pp.blocks[k].second == want) {
        void* p = pp.blocks[k].first;
        pp.blocks.erase(pp.blocks.begin() + (long)k);
        *cap = want;
        return p;
      }
    }
  }
  void* p = nullptr;
  hip_check(hipHostMalloc(&p, want, hipHostMallocDefault), "hipHostMalloc");
  *cap = want;
  return p;
}

void pinned_block_give(void* p, size_t cap) {
  if (!p) return;
  PendingPool& pp = pending_pool();
  std::lock_guard<std::mutex> lk(pp.mu);
  if (pp.blocks.size() < 64) {
    pp.blocks.emplace_back(p, cap);
    return;
  }
  (void)hipHostFree(p);
}

hipEvent_t pending_event_take(int device) {
  PendingPool& pp = pending_pool();
  {
    std::lock_guard<std::mutex> lk(pp.mu);
    for (size_t k = 0; k < pp.events.size(); ++k) {
      if (pp.events[k].first == device) {
        hipEvent_t e = pp.events[k].second;
        pp.events.erase(pp.events.begin() + (long)k);
        return e;
      }
    }
  }
  hipEvent_t e = nullptr;
  hip_check(hipEventCreateWithFlags(&e, hipEventDisableTiming), "hipEventCreateWithFlags");
  return e;
}

void pending_event_give(int device, hipEvent_t e) {
  if (!e) return;
  PendingPool& pp = pending_pool();
  std::lock_guard<std::mutex> lk(pp.mu);
  pp.events.emplace_back(device, e);
}

hipStream_t internal_stream(int device, int k) {
  if (k < 0 || k >= kInternalStreams) throw Error(TC_ERR_INTERNAL, "internal stream index out of range");
  static std::mutex mu;
  static std::vector<std::vector<hipStream_t>>* streams = new std::vector<std::vector<hipStream_t>>();
  std::lock_guard<std::mutex> lk(mu);
  if ((int)streams->size() <= device) streams->resize(device + 1);
  std::vector<hipStream_t>& v = (*streams)[device];
  while ((int)v.size() <= k) {
    hipStream_t st = nullptr;
    hip_check(hipStreamCreateWithFlags(&st, hipStreamNonBlocking), "hipStreamCreateWithFlags");
    v.push_back(st);
  }
  return v[k];
}

VoxTicket vox_slot_take(int device) {
  VoxPool& p = vox_pool();
  VoxTicket t{-1, nullptr, nullptr};
  {
    std::lock_guard<std::mutex> g(p.mu);
    for (size_t k = 0; k < p.idle.size(); ++k) {
      if (p.slots[p.idle[k]].device == device) {
        t.slot = p.idle[k];
        p.idle[k] = p.idle.back();
        p.idle.pop_back();
        break;
      }
    }
    if (t.slot < 0) {
      void* h = nullptr;
      hip_check(hipHostMalloc(&h, 64 * kVoxChunk, hipHostMallocDefault), "hipHostMalloc");
      const int base = (int)p.slots.size();
      for (int k = 0; k < kVoxChunk; ++k) {
        p.slots.push_back(VoxSlot{static_cast<int64_t*>(h) + 8 * k, nullptr, device});
        if (k) p.idle.push_back(base + k);
      }
      t.slot = base;
    }
    VoxSlot& v = p.slots[t.slot];
    if (!v.ev) hip_check(hipEventCreateWithFlags(&v.ev, hipEventDisableTiming), "hipEventCreateWithFlags");
    t.h = v.h;
    t.ev = v.ev;
  }
  // the slot's previous copy (its batch may have been freed unread) has landed
  if (hipEventQuery(t.ev) != hipSuccess) hip_check(hipEventSynchronize(t.ev), "hipEventSynchronize");
  return t;
}

void vox_slot_give(int slot) {
  if (slot < 0) return;
  VoxPool& p = vox_pool();
  std::lock_guard<std::mutex> g(p.mu);
  p.idle.push_back(slot);
}

// ------------------------------------------------------------------ profiling
namespace {
struct Timed {
  std::string name;
  hipEvent_t start, stop;
};
struct Prof {
  std::mutex mu;
  bool on = false;
  bool all = false;
  std::vector<std::string> names;
  std::vector<Timed> pending;
  std::vector<hipEvent_t> spare;  // events kept for reuse: creating one per launch costs host time
  hipEvent_t open_start = nullptr;
  std::vector<std::pair<std::string, std::pair<double, int64_t>>> totals;
  bool wants(const char* n) const {
    if (all) return true;
    for (const auto& x : names)
      if (x == n) return true;
    return false;
  }
};
Prof& prof() {
  static Prof* p = new Prof();
  return *p;
}

void prof_drain(Prof& p) {
  for (auto& t : p.pending) {
    hip_check(hipEventSynchronize(t.stop), "hipEventSynchronize");
    float ms = 0;
    hip_check(hipEventElapsedTime(&ms, t.start, t.stop), "hipEventElapsedTime");
    bool found = false;
    for (auto& kv : p.totals)
      if (kv.first == t.name) {
        kv.second.first += ms;
        kv.second.second += 1;
        found = true;
      }
    if (!found) p.totals.push_back({t.name, {(double)ms, 1}});
    p.spare.push_back(t.start);
    p.spare.push_back(t.stop);
  }
  p.pending.clear();
}

hipEvent_t take_event(Prof& p) {
  if (!p.spare.empty()) {
    hipEvent_t e = p.spare.back();
    p.spare.pop_back();
    return e;
  }
  hipEvent_t e;
  hip_check(hipEventCreate(&e), "hipEventCreate");
  return e;
}
}  // namespace

void prof_before(const char* name, hipStream_t s) {
  Prof& p = prof();
  if (!p.on) return;
  std::lock_guard<std::mutex> lk(p.mu);
  if (!p.on || !p.wants(name)) return;
  hipEvent_t e = take_event(p);
  hip_check(hipEventRecord(e, s), "hipEventRecord");
  p.open_start = e;
}

void prof_after(const char* name, hipStream_t s) {
  Prof& p = prof();
  if (!p.on) return;
  std::lock_guard<std::mutex> lk(p.mu);
  if (!p.on || !p.open_start || !p.wants(name)) return;
  hipEvent_t e = take_event(p);
  hip_check(hipEventRecord(e, s), "hipEventRecord");
  p.pending.push_back({name, p.open_start, e});
  p.open_start = nullptr;
}

void prof_enable(const char* names) {
  Prof& p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  for (auto& t : p.pending) {
    p.spare.push_back(t.start);
    p.spare.push_back(t.stop);
  }
  p.pending.clear();
  p.totals.clear();
  p.names.clear();
  p.all = std::strcmp(names, "*") == 0;
  std::string cur;
  for (const char* c = names;; ++c) {
    if (*c == ',' || *c == 0) {
      if (!cur.empty()) p.names.push_back(cur);
      cur.clear();
      if (*c == 0) break;
    } else if (*c != ' ') {
      cur.push_back(*c);
    }
  }
  while (p.spare.size() < 1024) {  // enough for a timed loop without creating events in it
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) {  // no device here: events are created when needed
      (void)hipGetLastError();
      break;
    }
    p.spare.push_back(e);
  }
  p.on = true;
}

void prof_read(const char* name, double* ms, int64_t* n) {
  Prof& p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  prof_drain(p);
  *ms = 0;
  *n = 0;
  for (auto& kv : p.totals)
    if (kv.first == name) {
      *ms = kv.second.first;
      *n = kv.second.second;
    }
}

void prof_disable() {
  Prof& p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  prof_drain(p);
  p.on = false;
}

}  // namespace tc
