// Internal declarations shared by the HIP translation units of the library.
// Not part of the public ABI (see include/topo.h).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <stdexcept>
#include <string>
#include <vector>

#include "../../include/topo.h"

namespace tc {

using u64 = uint64_t;
using i64 = int64_t;

// ------------------------------------------------------------------ errors
struct Error : std::runtime_error {
  tc_status status;
  Error(tc_status s, const std::string& msg) : std::runtime_error(msg), status(s) {}
};

inline void hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess)
    throw Error(TC_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// ------------------------------------------------------------------ op tables
// Per-axis offset sets of the box ops (PR page section 2): DILATE {-1,0,1},
// PAD_NEG {-1,0}, PAD_POS {0,1}. `m` = number of neighbour combinations; j in
// [0, m) enumerates them x-major.
struct OpInfo {
  int op;
  int m;       // candidate targets per source node (tiles per upper, lowers per lower)
  int m_src;   // source lowers that can feed one candidate lower
  int lo, hi;  // box offset range per axis (box ops only)
};

inline OpInfo op_info(int op) {
  switch (op) {
    case TC_OP_REFINE: return {op, 8, 1, 0, 0};
    case TC_OP_COARSEN: return {op, 1, 8, 0, 0};
    case TC_OP_DILATE: return {op, 27, 27, -1, 1};
    case TC_OP_PAD_NEG: return {op, 8, 27, -1, 0};
    case TC_OP_PAD_POS: return {op, 8, 27, 0, 1};
    default: throw Error(TC_ERR_INVALID_ARG, "unknown op");
  }
}

// ------------------------------------------------------------------ layout
struct Layout {
  size_t headers, status, upper_origin, upper_key, upper_first, upper_mask, lower_origin, lower_first,
      lower_mask, lower_prefix, leaf_origin, leaf_parent, leaf_mask, leaf_prefix, leaf_offset;
  size_t total;
};

inline size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

inline Layout make_layout(i64 B, i64 n2, i64 n1, i64 nl) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  // the B headers, then a 16-byte status word (int32 flags of the writer
  // kernels, then zeros) that is read back together with the last header
  L.headers = take(sizeof(tc_grid_header) * (size_t)B + 16);
  L.status = L.headers + sizeof(tc_grid_header) * (size_t)B;
  L.upper_origin = take(16 * (size_t)n2);
  L.upper_key = take(8 * (size_t)n2);
  L.upper_first = take(4 * (size_t)n2);
  L.upper_mask = take(4096 * (size_t)n2);
  L.lower_origin = take(16 * (size_t)n1);
  L.lower_first = take(4 * (size_t)n1);
  L.lower_mask = take(512 * (size_t)n1);
  L.lower_prefix = take(128 * (size_t)n1);
  L.leaf_origin = take(16 * (size_t)nl);
  L.leaf_parent = take(4 * (size_t)nl);
  L.leaf_mask = take(64 * (size_t)nl);
  L.leaf_prefix = take(8 * (size_t)nl);
  L.leaf_offset = take(8 * (size_t)nl);
  L.total = off;
  return L;
}

// Device views of a grid batch (all pointers into its single buffer).
struct GridView {
  int32_t B, n_upper, n_lower, n_leaf;
  tc_grid_header* headers;
  int32_t* status;  // [4]: writer flags (non-zero: a failed consistency check), 0, 0, 0
  int4* upper_origin;
  u64* upper_key;
  int32_t* upper_first;
  u64* upper_mask;
  int4* lower_origin;
  int32_t* lower_first;
  u64* lower_mask;
  uint16_t* lower_prefix;
  int4* leaf_origin;
  int32_t* leaf_parent;
  u64* leaf_mask;
  u64* leaf_prefix;
  i64* leaf_offset;
};

inline GridView make_view(void* buffer, const Layout& L, int32_t B, int32_t n2, int32_t n1, int32_t nl) {
  char* b = static_cast<char*>(buffer);
  GridView v;
  v.B = B;
  v.n_upper = n2;
  v.n_lower = n1;
  v.n_leaf = nl;
  v.headers = reinterpret_cast<tc_grid_header*>(b + L.headers);
  v.status = reinterpret_cast<int32_t*>(b + L.status);
  v.upper_origin = reinterpret_cast<int4*>(b + L.upper_origin);
  v.upper_key = reinterpret_cast<u64*>(b + L.upper_key);
  v.upper_first = reinterpret_cast<int32_t*>(b + L.upper_first);
  v.upper_mask = reinterpret_cast<u64*>(b + L.upper_mask);
  v.lower_origin = reinterpret_cast<int4*>(b + L.lower_origin);
  v.lower_first = reinterpret_cast<int32_t*>(b + L.lower_first);
  v.lower_mask = reinterpret_cast<u64*>(b + L.lower_mask);
  v.lower_prefix = reinterpret_cast<uint16_t*>(b + L.lower_prefix);
  v.leaf_origin = reinterpret_cast<int4*>(b + L.leaf_origin);
  v.leaf_parent = reinterpret_cast<int32_t*>(b + L.leaf_parent);
  v.leaf_mask = reinterpret_cast<u64*>(b + L.leaf_mask);
  v.leaf_prefix = reinterpret_cast<u64*>(b + L.leaf_prefix);
  v.leaf_offset = reinterpret_cast<i64*>(b + L.leaf_offset);
  return v;
}

// ------------------------------------------------------------------ host-side memory
// Where a call's device memory comes from: the allocator given to its entry
// point, or (NULL) the device's stream-ordered pool. Set for the calling thread
// for the duration of the scope; arenas and intermediate batches use it.
class SourceScope {
 public:
  explicit SourceScope(const tc_allocator* a);
  ~SourceScope();
  SourceScope(const SourceScope&) = delete;
  SourceScope& operator=(const SourceScope&) = delete;

 private:
  tc_allocator prev_;
  bool prev_set_;
};

// Scratch blocks cached per (device, stream, source), process-wide: a block is
// taken by one arena (or one intermediate batch) at a time and given back
// without being freed, so reuse is ordered by its stream. scratch_release_all()
// frees every idle block (after a device synchronisation).
struct ScratchBlock;
ScratchBlock* scratch_acquire(size_t bytes, hipStream_t s);
void scratch_give_back(ScratchBlock* b, hipStream_t s);
char* scratch_ptr(const ScratchBlock* b);
void scratch_release_all();
size_t scratch_cached_bytes();

// Scratch arena: one block carved into 256-byte aligned arrays. The block comes
// from the scratch cache (current source) and returns to it when the arena is
// destroyed.
class Arena {
 public:
  explicit Arena(hipStream_t s) : stream_(s) {}
  ~Arena() { release(); }
  Arena(const Arena&) = delete;
  Arena& operator=(const Arena&) = delete;
  // Reserve `bytes` (rounded up); returns an offset handle resolved after commit().
  size_t reserve(size_t bytes) {
    size_t at = size_;
    size_ = align_up(size_ + (bytes ? bytes : 1));
    return at;
  }
  void commit();
  template <typename T>
  T* at(size_t off) const { return reinterpret_cast<T*>(base_ + off); }
  void release();
  size_t size() const { return size_; }

 private:
  hipStream_t stream_;
  char* base_ = nullptr;
  size_t size_ = 0;
  ScratchBlock* block_ = nullptr;
};

// Buffers of batches built without an allocator, cached per device and stream
// between tc_batch_free and the next batch that fits (capacity in *cap).
void* batch_buffer_take(size_t bytes, hipStream_t s, size_t* cap);
void batch_buffer_give(void* p, size_t cap, int device, hipStream_t s);
void batch_buffers_release();

// Compute units of the current device (read once per device).
int device_cu_count();

// Per-thread pinned host staging buffer (grows on demand, never shrinks).
void* pinned_staging(size_t bytes);

// Pinned 64-byte host slots, each with an event, for the tail of a batch's last
// header and its status word (int64 words 0 and 1: the last grid's voxel count
// and begin; word 6: the writer flags): the copy is queued behind a builder's
// last kernel and read when first asked. Slots belong to a device; taking one
// waits for its previous copy to land.
struct VoxTicket {
  int slot;
  int64_t* h;
  hipEvent_t ev;
};
VoxTicket vox_slot_take(int device);
void vox_slot_give(int slot);

// Pinned host blocks and events for batches whose headers are still being read
// back (pooled; a block's size is the power of two >= bytes, at least 4 KiB).
void* pinned_block_take(size_t bytes, size_t* cap);
void pinned_block_give(void* p, size_t cap);
hipEvent_t pending_event_take(int device);
// Internal stream k (0 <= k < kInternalStreams) of the current device: created
// once, non-blocking, default priority, kept until the process ends.
constexpr int kInternalStreams = 4;
constexpr int kSideStreams = 1;  // internal streams a multi-target build spreads its targets over
hipStream_t internal_stream(int device, int k);
void pending_event_give(int device, hipEvent_t e);

// Stream-ordered device allocation from the device's default pool (release
// threshold raised once per device so that memory is cached across calls).
void* device_alloc_async(size_t bytes, hipStream_t s);
void device_free_async(void* p, hipStream_t s);

// ------------------------------------------------------------------ profiling
// When `name` is being timed, prof_before records a start event on the stream
// and prof_after a stop event; the pair is read later (prof_read). The interval
// includes the dispatch latency between the start marker and the kernel.
void prof_before(const char* name, hipStream_t s);
void prof_after(const char* name, hipStream_t s);

template <typename Kernel, typename... Args>
inline void launch(const char* name, Kernel kernel, i64 blocks, int threads, hipStream_t s, Args... args) {
  if (blocks <= 0) return;
  if (blocks > 0x7fffffffLL) throw Error(TC_ERR_UNSUPPORTED, std::string(name) + ": grid too large");
  prof_before(name, s);
  hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(threads), 0, s, args...);
  hip_check(hipGetLastError(), name);
  prof_after(name, s);
}

// As launch(), with `lds_bytes` of dynamic shared memory.
template <typename Kernel, typename... Args>
inline void launch_lds(const char* name, Kernel kernel, i64 blocks, int threads, size_t lds_bytes, hipStream_t s,
                       Args... args) {
  if (blocks <= 0) return;
  if (blocks > 0x7fffffffLL) throw Error(TC_ERR_UNSUPPORTED, std::string(name) + ": grid too large");
  prof_before(name, s);
  hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(threads), lds_bytes, s, args...);
  hip_check(hipGetLastError(), name);
  prof_after(name, s);
}

inline i64 ceil_div(i64 a, i64 b) { return (a + b - 1) / b; }

// ------------------------------------------------------------------ primitives (primitives.hip)
// Exclusive scan of n items (n read from d_n when non-null, else n_host; n_host
// is the launch bound). out has n+1 entries; out[n] = total.
// total_out, when given, also receives the total (device memory). Scans longer
// than one tile need scan_tmp_bytes(n_host, sizeof(T)) of scratch: from `tmp`
// when given, else allocated (and freed) on the stream.
size_t scan_tmp_bytes(i64 n_host, size_t elem);
void scan_excl_i32(const int32_t* in, int32_t* out, i64 n_host, const int32_t* d_n, hipStream_t s,
                   int32_t* total_out = nullptr, void* tmp = nullptr);
void scan_excl_i64(const i64* in, i64* out, i64 n_host, const int32_t* d_n, hipStream_t s,
                   i64* total_out = nullptr, void* tmp = nullptr);
void scan_excl_u32(const uint32_t* in, uint32_t* out, i64 n_host, const int32_t* d_n, hipStream_t s);

void fill_i32(int32_t* p, int32_t v, i64 n_host, const int32_t* d_n, int32_t mult, hipStream_t s);
void fill_u64(u64* p, u64 v, i64 n_host, const int32_t* d_n, int32_t mult, hipStream_t s);
void fill_pair(int32_t* a, int32_t va, i64 na_host, int32_t mult_a, u64* b, u64 vb, i64 nb_host, int32_t mult_b,
               const int32_t* d_n, hipStream_t s);

// Sorts (key_hi, key_lo) 128-bit keys with uint32 values ascending. `key_bits`
// bounds the significant low bits of every key (keys above them compare by
// those bits only). n is host-known.
struct Key128 {
  u64 lo, hi;
};
void sort_pairs_128(Key128* keys, uint32_t* vals, i64 n, int key_bits, hipStream_t s);

// Bits of a builder's device flag word (copied into the batch's status word).
constexpr int kFlagOverflow = 1;
constexpr int kFlagInternal = 2;  // a consistency check of a kernel failed
constexpr int kFlagSource = 4;    // the source batch's writers had flagged a failed check

// ------------------------------------------------------------------ tile keys
// A tile key packs (grid, Tx+2^19, Ty+2^19, Tz+2^19) as grid<<60 | tx<<40 | ty<<20 | tz
// over 128 bits; INVALID sorts after every valid key.
constexpr int kTileBias = 1 << 19;
inline int tile_key_bits(int32_t B) {
  int gb = 0;
  while (gb < 31 && ((int64_t)1 << gb) < B) ++gb;
  return 61 + gb;  // one spare bit keeps INVALID above every valid key
}

// ------------------------------------------------------------------ tree assembly (tree.hip)
// Candidate-node state shared by the topology pass and the ijk front-end.
struct TreeScratch {
  // tiles (unique, canonical order)
  int32_t* d_num_tiles;      // [1]
  int4* utile;               // [cap_tiles] Tx, Ty, Tz, grid
  u64* tile_child;           // [cap_tiles][512]
  uint16_t* tile_prefix;     // [cap_tiles][512]
  int32_t* tile_lower_count; // [cap_tiles]
  int32_t* tile_lower_base;  // [cap_tiles + 1]
  int32_t* tile_nonempty;    // [cap_tiles]
  int32_t* upper_excl;       // [cap_tiles + 1]
  int32_t* grid_tile_begin;  // [B + 1]
  // candidate lowers
  int32_t* d_num_cands;      // [1] candidate lowers (total of the tile scan)
  int4* cand_origin;         // [cap_cands] x, y, z (voxel origin), tile
  u64* cand_child;           // [cap_cands][64]
  uint16_t* cand_prefix;     // [cap_cands][64]
  i64* cand_counts;          // [cap_cands] leaf count | non-empty << 32
  i64* cand_scan;            // [cap_cands + 1] exclusive scan: first leaf | output lower index << 32
  // per-grid results
  int32_t* grid_info;        // [B][6]: nU, nL1, nL, uBegin, lBegin, leafBegin
  int32_t* readback;         // [4 + 3B]: flags, N2, N1, L, then per-grid counts
  int32_t* flags;            // [1] bit 0 overflow, bit 1 internal error (inside readback)
  void* scan_tmp;            // scan scratch: scan_tmp_bytes over cap_tiles (i32) and cap_cands (i64)
  i64 cap_tiles, cap_cands;
  bool cand_counts_ready;    // the marking wrote cand_prefix and cand_counts (else the counts stage does)
};

// Launch groups (implemented in tree.hip).
void tree_tile_ranges(TreeScratch& t, int32_t B, hipStream_t s);
// The counts stages below also write the readback words (flag word, totals,
// per-grid counts) to `host_rb` (pinned host memory, or null) when one
// workgroup computes them all; they return whether they did, else the caller
// copies the words back itself.
bool tree_grid_counts(TreeScratch& t, int32_t B, hipStream_t s, int32_t* host_rb = nullptr);
void tree_rank_tiles(TreeScratch& t, hipStream_t s);
// tree_rank_tiles and the candidate -> source table's fill (nc * m_src entries
// of cand_src set to -1) in one launch, for at most 4096 tile slots; done_ctr is
// a device word zeroed before the launch (by the tile stage).
void tree_rank_tiles_last(TreeScratch& t, int32_t* done_ctr, int32_t* cand_src, int32_t m_src, hipStream_t s);            // prefix per tile + scan -> cand numbering
void tree_count_cands(TreeScratch& t, hipStream_t s);           // leaf counts per cand + their scan
bool tree_counts(TreeScratch& t, int32_t B, hipStream_t s, int32_t* host_rb = nullptr);  // tree_count_cands + tree_grid_counts (fused when small)
void tree_write_nodes(TreeScratch& t, const GridView& out, int32_t* leaf_cand, hipStream_t s);
// tree_counts and tree_write_nodes in one launch, for at most 2048 candidate and
// tile slots once the marking wrote the candidates' counts (..._fits says when).
bool write_nodes_counted_fits(const TreeScratch& t, int32_t B);
void tree_write_nodes_counted(TreeScratch& t, const GridView& out, int32_t* leaf_cand, hipStream_t s);
// Leaf masks from eight word slices (slice k: word k of every leaf), and their
// statistics.
void tree_leaf_stats(const GridView& out, const u64* slices, uint32_t* leaf_box, int32_t* leaf_inrun, i64* vox_part,
                     hipStream_t s);
int32_t bbox_replicas(int32_t B);  // replicas of the per-grid bbox accumulators
// Leaf voxel offsets, per-grid bboxes and headers. The leaf producer wrote, per
// run of `gran` leaves (gran divides 256), the run's voxel sum (vox_part) and
// every leaf's voxels before it inside its run (leaf_inrun).
// `flags` is the builder's flag word; its final value goes to out.status.
// d_L (device) holds the leaf count; out.n_leaf is that count, or a capacity
// above it when the batch's arrays were laid out by capacities (small path only).
// With host_words (pinned host memory of at least B headers + 16 bytes) the
// one-launch finalize's workgroup 0 also writes there every header's counts and
// begins (not its box) and, after the headers, the status word.
void tree_finalize_leaves(const GridView& out, const uint32_t* leaf_box, const int32_t* leaf_inrun, i64* vox_part,
                          i64 gran, i64* gvb, int32_t* bbox_accum, const int32_t* grid_info, int32_t* flags,
                          const int32_t* d_L, hipStream_t s, int32_t* host_words = nullptr);
// Whether the one-launch finalize takes L leaves (or a capacity of L) of B grids.
bool finalize_small_fits(i64 L, int32_t B, i64 gran);
void tree_enumerate(const GridView& v, int32_t* ijk, hipStream_t s);
// tree_enumerate of n batches (output ijk[j] for batch j), up to eight per launch.
void tree_enumerate_many(const GridView* v, int32_t* const* ijk, int n, hipStream_t s);

// Allocation of the single output buffer of a batch.
struct OutAlloc {
  const tc_allocator* alloc;  // NULL: the library's own (hipMallocAsync, cached)
  hipStream_t stream;         // the stream the pass's work is enqueued on
  bool transient = false;     // an intermediate batch of a chain: a scratch block of the call's source
  // when set, the output's buffer is taken on (and later handed back on) this
  // stream instead: the caller's stream, for outputs built on an internal stream
  // whose work the caller's stream waits for
  hipStream_t alloc_stream = nullptr;
};

// Testing: bits that the next batch built on the calling thread ORs into its
// writers' device flag word (tc_debug_inject_flags); apply_debug_inject sets
// them (once) on the flag word of the batch being built, before its finalize.
void debug_set_inject(int32_t bits);
void apply_debug_inject(int32_t* d_flags, hipStream_t s);
// Testing: while set on the calling thread, the box ops' leaf gather takes its
// 64-bit-address form (the one batches with source arrays of 2 GiB or more use).
void debug_set_wide_loads(bool on);
bool debug_wide_loads();

void prof_enable(const char* name);
void prof_read(const char* name, double* ms, int64_t* n);
void prof_disable();

}  // namespace tc

// The opaque batch handle of the C ABI.
struct tc_grid_batch {
  int32_t B = 0, n2 = 0, n1 = 0, nl = 0;
  std::vector<int32_t> h_upper, h_lower, h_leaf;
  void* buffer = nullptr;
  size_t bytes = 0;
  size_t cap = 0;  // buffer capacity when the library allocated it
  tc::Layout layout{};
  bool has_alloc = false;
  tc_allocator alloc{};
  tc::ScratchBlock* block = nullptr;  // the buffer of an intermediate batch (scratch cache)
  hipStream_t stream = nullptr;
  int device = 0;
  mutable bool vox_known = false;
  mutable int64_t vox_total = 0;
  // voxel total and status word queued for readback (queue_voxel_total): slot,
  // host words, event
  mutable bool vox_pending = false;
  mutable bool status_bad = false;  // a writer kernel's device consistency check failed
  mutable int vox_slot = -1;
  mutable int64_t* vox_h = nullptr;
  mutable hipEvent_t vox_ev = nullptr;
  // a small batch built with its headers still on their way (a pass of
  // tc_build_batched_topology_many): its finalize writes every header's counts
  // and the status word into hdr_host, and hdr_ev follows that kernel; the counts
  // are set by resolve_counts
  mutable bool hdr_pending = false;
  mutable void* hdr_host = nullptr;
  mutable size_t hdr_host_cap = 0;
  mutable hipEvent_t hdr_ev = nullptr;

  tc::GridView view() const {
    return tc::make_view(buffer, layout, B, n2, n1, nl);
  }
};

namespace tc {
// Creates the output batch from the readback of a tree assembly (counts per
// grid) and allocates its buffer; throws on failure (nothing leaked).
tc_grid_batch* new_batch(int32_t B, const int32_t* readback, const OutAlloc& oa);
// A batch whose arrays are laid out by capacities (counts set later from its
// headers by set_counts_from_headers, which also makes the voxel total known).
tc_grid_batch* new_batch_capacity(int32_t B, i64 n2_cap, i64 n1_cap, i64 nl_cap, const OutAlloc& oa);
void set_counts_from_headers(tc_grid_batch* b, const tc_grid_header* h);
void free_batch(tc_grid_batch* b);
tc_grid_batch* copy_batch(const tc_grid_batch* src, const OutAlloc& oa);  // same counts, one D2D copy
// Throws TC_ERR_INTERNAL when the batch's writers flagged a failed consistency
// check (the status word comes back with the voxel total: this waits for that
// copy the first time).
void check_status(const tc_grid_batch* b);
// Kernel map of `dst` against `src` (same member count): out int32[V_dst][K^3],
// `entries` = V_dst * K^3. Scratch from an arena, or from `scratch` (device,
// scratch_cap bytes, at least kernel_map_scratch_bytes) when given.
void kernel_map(const GridView& src, const GridView& dst, int K, int S, int transposed, int32_t* out, i64 entries,
                hipStream_t s, char* scratch = nullptr, size_t scratch_cap = 0);
size_t kernel_map_scratch_bytes(const GridView& src, const GridView& dst, int K, int S, int transposed);
// Device address of the current GPU's static no-allocation scratch array and
// its size (hipGetSymbolAddress once per device).
char* noalloc_scratch(size_t* cap);

// The two producers of grid batches.
tc_grid_batch* build_from_ijk(const int32_t* d_ijk, const int64_t* h_offsets, int32_t B, const OutAlloc& oa);
// Points front-end: float32 points -> voxel rows (mode 0: nearest voxel centre,
// mode 1: the 8 surrounding voxels) -> build_from_ijk.
tc_grid_batch* build_from_points(const float* d_xyz, const int64_t* h_offsets, int32_t B, const float* h_voxel_size,
                                 const float* h_origin, int mode, const OutAlloc& oa);
// One batched pass. leaf_mask_override (device, one 512-bit mask per source leaf)
// replaces the source leaf masks, e.g. masked copies for masked refine.
// Waits for a pending batch's headers (hdr_pending) and sets its counts from
// them; throws on a flagged pass (the batch stays to be freed by its owner).
void resolve_counts(const tc_grid_batch* b);
// With `defer`, a small batch's pass returns with its headers pending (see
// tc_grid_batch::hdr_pending); the caller resolves them (resolve_counts).
tc_grid_batch* build_pass(const tc_grid_batch* src, int op, const OutAlloc& oa,
                          const u64* leaf_mask_override = nullptr, bool defer = false);
// Masked copies of src's leaf masks from per-voxel keep flags (enumeration order);
// a flag index outside [0, n_keep) sets the internal-error bit in *flags.
void mask_leaves(const tc_grid_batch* src, const uint8_t* keep, i64 n_keep, u64* out_mask, int32_t* flags,
                 hipStream_t s);
}  // namespace tc
