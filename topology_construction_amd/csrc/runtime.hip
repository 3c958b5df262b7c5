// Host runtime helpers: stream-ordered scratch memory, pinned staging buffers,
// kernel timing with HIP events.
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

void Arena::commit() {
  if (base_) throw Error(TC_ERR_INTERNAL, "arena committed twice");
  base_ = static_cast<char*>(device_alloc_async(size_, stream_));
}

void Arena::release() {
  if (base_) device_free_async(base_, stream_);
  base_ = nullptr;
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

// ------------------------------------------------------------------ profiling
namespace {
struct Prof {
  std::mutex mu;
  bool on = false;
  std::string name;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pending;
  hipEvent_t open_start = nullptr;
  double total_ms = 0;
  int64_t launches = 0;
};
Prof& prof() {
  static Prof* p = new Prof();
  return *p;
}
}  // namespace

void prof_before(const char* name, hipStream_t s) {
  Prof& p = prof();
  if (!p.on) return;
  std::lock_guard<std::mutex> lk(p.mu);
  if (!p.on || p.name != name) return;
  hipEvent_t e;
  hip_check(hipEventCreate(&e), "hipEventCreate");
  hip_check(hipEventRecord(e, s), "hipEventRecord");
  p.open_start = e;
}

void prof_after(const char* name, hipStream_t s) {
  Prof& p = prof();
  if (!p.on) return;
  std::lock_guard<std::mutex> lk(p.mu);
  if (!p.on || p.name != name || !p.open_start) return;
  hipEvent_t e;
  hip_check(hipEventCreate(&e), "hipEventCreate");
  hip_check(hipEventRecord(e, s), "hipEventRecord");
  p.pending.emplace_back(p.open_start, e);
  p.open_start = nullptr;
}

static void prof_drain(Prof& p) {
  for (auto& pr : p.pending) {
    hip_check(hipEventSynchronize(pr.second), "hipEventSynchronize");
    float ms = 0;
    hip_check(hipEventElapsedTime(&ms, pr.first, pr.second), "hipEventElapsedTime");
    p.total_ms += ms;
    p.launches += 1;
    (void)hipEventDestroy(pr.first);
    (void)hipEventDestroy(pr.second);
  }
  p.pending.clear();
}

void prof_enable(const char* name) {
  Prof& p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  for (auto& pr : p.pending) {
    (void)hipEventDestroy(pr.first);
    (void)hipEventDestroy(pr.second);
  }
  p.pending.clear();
  p.name = name;
  p.total_ms = 0;
  p.launches = 0;
  p.on = true;
}

void prof_read(double* ms, int64_t* n) {
  Prof& p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  prof_drain(p);
  *ms = p.total_ms;
  *n = p.launches;
}

void prof_disable() {
  Prof& p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  prof_drain(p);
  p.on = false;
}

}  // namespace tc
