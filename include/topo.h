/*
 * topo.h -- C ABI of the batched generated-topology library for MI355X (gfx950).
 *
 * The library builds, for a batch of B sparse voxel grids at once, the topology
 * of a generated grid: coarsen by 2/4/8, refine by 2/4/8, box-dilate [-1,1]^3,
 * pad {-1,0}^3 or {0,1}^3, and the k3s2 transposed-conv target (refine by 2 then
 * pad {-1,0}^3). Each grid is a three-level tree of 8^3 leaves (512-bit active
 * masks), 16^3-leaf lower nodes, 32^3-lower upper nodes and one root tile per
 * upper node, stored in the canonical x-major tree order. One pass runs over all
 * source leaves of all members, with one host readback of node counts.
 *
 * Source of the operations and outputs: the fvdb-core pages
 *   - "Generated-topology grid construction dominates per-iteration
 *     ConvolutionPlan cost" (issue page): Summary, Root cause, Suggested direction;
 *   - "Batched leaf-mask topology construction for generated conv grids"
 *     (PR page): section 1 (one emission pass, canonical order, dedup, one
 *     readback, batched writers, empty members, multi-pass factors 4 and 8),
 *     section 2 (box-dilate passes, pads, k3s2 transpose), Test plan.
 *
 * Conventions (all entry points):
 *   - Pointers named d_* are HIP device pointers; h_* are host pointers.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream). All device
 *     work is enqueued on it; device outputs become valid in stream order.
 *   - Every entry point validates its arguments on the host before any launch.
 *     On any non-TC_OK status, *out is set to NULL, nothing is leaked and
 *     tc_last_error() returns a message for the calling thread.
 *   - int32 overflow of an output coordinate is detected on the device, by the
 *     kernels that compute the output nodes, and reported at the pass's one
 *     readback (TC_ERR_OVERFLOW, no batch), before any output is allocated.
 *   - The kernels that write a batch's leaf masks check their indices; a failed
 *     check (a library defect, never an input property) is reported as
 *     TC_ERR_INTERNAL: by the pass itself when it ends on the readback of the
 *     batch's headers (small batches, see tc_build_batched_topology), else by
 *     the first call that blocks on the batch afterwards (tc_batch_voxel_total,
 *     tc_batch_read_headers, tc_enumerate_ijk, tc_build_kernel_map, or a pass
 *     that reads it), and by every later one.
 *   - Calls on different streams or threads are independent. A tc_grid_batch is
 *     immutable after creation and may be read concurrently.
 *   - Coordinates are int32 voxel indices; counts are int32 (nodes) or int64
 *     (voxels).
 */
#ifndef TOPO_H
#define TOPO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TC_ABI_VERSION 1

typedef enum tc_status {
  TC_OK = 0,
  TC_ERR_INVALID_ARG = 1,  /* bad pointer, op, factor, B < 1, bad offsets, capacity */
  TC_ERR_OVERFLOW = 2,     /* an output voxel coordinate would leave int32 */
  TC_ERR_ALLOC = 3,        /* the allocator (or the HIP pool) returned no memory */
  TC_ERR_HIP = 4,          /* a HIP runtime call failed; message has the HIP error */
  TC_ERR_UNSUPPORTED = 5,  /* e.g. a factor that is not a power of two */
  TC_ERR_INTERNAL = 6      /* a device-side consistency check failed */
} tc_status;

/* Operations (PR page sections 1 and 2).
 *   TC_OP_COARSEN     factor 2, 4 or 8: { floor(v / f) }         (conv_grid k2s2 for f = 2)
 *   TC_OP_REFINE      factor 2, 4 or 8: { f*v + d, d in [0,f)^3 } (conv_transpose_grid k2s2)
 *   TC_OP_DILATE      factor 1: Minkowski sum with [-1,1]^3       (conv_grid k3s1)
 *   TC_OP_PAD_NEG     factor 1: Minkowski sum with {-1,0}^3
 *   TC_OP_PAD_POS     factor 1: Minkowski sum with {0,1}^3
 *   TC_OP_CONV_T_K3S2 factor 2: refine by 2, then TC_OP_PAD_NEG   (conv_transpose_grid k3s2)
 *   TC_OP_CONV_S1     factor K in [1,8]: Minkowski sum with [-floor(K/2), floor((K-1)/2)]^3
 *                     (conv_grid, kernel K, stride 1)
 *   TC_OP_CONV_T_S1   factor K in [1,8]: Minkowski sum with [-floor((K-1)/2), floor(K/2)]^3
 *                     (conv_transpose_grid, kernel K, stride 1)
 * Factors 4 and 8 (and k3s2) run chained x2 passes, each with its own readback.
 * The kernel-K ops run as sequences of TC_OP_DILATE / TC_OP_PAD_* passes (PR page
 * section 2; K in {2,3,4,5} in its test plan): the kernel's offsets are
 * [-floor((K-1)/2), floor(K/2)] per axis, the transposed conv scatters to them and
 * the conv gathers from them; K = 1 returns a copy of the source.
 * Coarsening rounds toward minus infinity. */
typedef enum tc_op {
  TC_OP_COARSEN = 1,
  TC_OP_REFINE = 2,
  TC_OP_DILATE = 3,
  TC_OP_PAD_NEG = 4,
  TC_OP_PAD_POS = 5,
  TC_OP_CONV_T_K3S2 = 6,
  TC_OP_CONV_S1 = 7,
  TC_OP_CONV_T_S1 = 8
} tc_op;

/* Caller-supplied device allocator. When an entry point is given one, all the
 * device memory of that call comes from it: the output batch's buffer (one
 * allocation per output batch, returned through `free` by tc_batch_free), the
 * scratch arrays of the passes and the intermediate batches of chained passes.
 * `alloc` returns a device pointer usable on `stream`, aligned to at least 256
 * bytes, or NULL on failure (the call then fails with TC_ERR_ALLOC, *out is NULL
 * and nothing is leaked). `free` receives the same pointer, byte count and
 * stream. Both are called from the thread that calls into the library (or, for
 * cached scratch, from the thread of a later call or of tc_scratch_release).
 * Scratch blocks are not freed at the end of a call: the library caches them
 * per (device, stream, allocator) and hands them to the next call with the
 * same key, so a steady stream of passes makes no allocator calls beyond its
 * outputs; tc_scratch_release returns the idle ones through `free`.
 * Passing a NULL tc_allocator* makes the library take all of this from the
 * device's stream-ordered pool (hipMallocAsync on the call's stream), with
 * the same caching. */
typedef struct tc_allocator {
  void* (*alloc)(void* ctx, size_t bytes, void* stream);
  void (*free)(void* ctx, void* ptr, size_t bytes, void* stream);
  void* ctx;
} tc_allocator;

typedef struct tc_grid_batch tc_grid_batch; /* opaque, owned by the caller */

/* Per-grid header (PR page section 1: every grid gets mGridIndex = g,
 * mGridCount = B, its node counts and its bbox). 80 bytes, device resident. */
typedef struct tc_grid_header {
  int32_t grid_index;   /* g */
  int32_t grid_count;   /* B */
  int32_t upper_count;  /* upper nodes (= root tiles) of this grid */
  int32_t lower_count;
  int32_t leaf_count;
  int32_t upper_begin;  /* batch-global index of the grid's first upper node */
  int32_t lower_begin;
  int32_t leaf_begin;
  int64_t voxel_count;
  int64_t voxel_begin;  /* batch-global index of the grid's first voxel */
  int32_t bbox_min[3];  /* inclusive index-space bbox of active voxels; an empty */
  int32_t bbox_max[3];  /* grid has min = INT32_MAX and max = INT32_MIN */
  int32_t reserved[2];
} tc_grid_header;

/* Device arrays of a batch, all inside one allocation (`buffer`), in canonical
 * order: grids in order; inside a grid root tiles by signed x-major tile
 * coordinate, then x-major child offsets. Layouts:
 *   upper_origin int32[N2][4]  x, y, z (multiple of 4096), grid
 *   upper_key    uint64[N2]    (Tx+2^19)<<40 | (Ty+2^19)<<20 | (Tz+2^19), T = origin/4096
 *   upper_first  int32[N2]     index of the first child lower node
 *   upper_mask   uint64[N2][512] child bit (x*32+y)*32+z of the lower inside the upper
 *   lower_origin int32[N1][4]  x, y, z (multiple of 128), parent upper index
 *   lower_first  int32[N1]     index of the first child leaf
 *   lower_mask   uint64[N1][64]  child bit (x*16+y)*16+z of the leaf inside the lower
 *   lower_prefix uint16[N1][64]  active children in words < w
 *   leaf_origin  int32[L][4]   x, y, z (multiple of 8), grid
 *   leaf_parent  int32[L]      parent lower index
 *   leaf_mask    uint64[L][8]  voxel bit n = x*64 + y*8 + z (word x, bit y*8+z)
 *   leaf_prefix  uint64[L]     seven 9-bit fields; field w-1 = voxels in words < w
 *   leaf_offset  int64[L]      0-based index of the leaf's first voxel in its grid
 * Node indices are batch-global. */
typedef struct tc_batch_info {
  int32_t grid_count;
  int32_t upper_count;
  int32_t lower_count;
  int32_t leaf_count;
  const int32_t* h_upper_counts; /* [B], host, valid for the batch's lifetime */
  const int32_t* h_lower_counts;
  const int32_t* h_leaf_counts;
  const void* d_buffer;
  size_t buffer_bytes;
  const tc_grid_header* d_headers;
  const int32_t* d_upper_origin;
  const uint64_t* d_upper_key;
  const int32_t* d_upper_first;
  const uint64_t* d_upper_mask;
  const int32_t* d_lower_origin;
  const int32_t* d_lower_first;
  const uint64_t* d_lower_mask;
  const uint16_t* d_lower_prefix;
  const int32_t* d_leaf_origin;
  const int32_t* d_leaf_parent;
  const uint64_t* d_leaf_mask;
  const uint64_t* d_leaf_prefix;
  const int64_t* d_leaf_offset;
} tc_batch_info;

/* Library version of this header; a caller checks it equals TC_ABI_VERSION. */
int32_t tc_abi_version(void);

/* Static text for a status code. */
const char* tc_status_string(tc_status status);

/* Message describing the calling thread's most recent non-TC_OK status. */
const char* tc_last_error(void);

/* Builds a batch of B grids from int32 voxel rows (the ijk front-end; PR page,
 * Measurements: follow-up ijk emission front-end, and Test plan: expected
 * topologies built from ijk).
 *   d_ijk      int32[N][3] device, N = h_offsets[B]; may be NULL when N = 0.
 *   h_offsets  int64[B+1] host: member g owns rows [h_offsets[g], h_offsets[g+1]);
 *              h_offsets[0] = 0, non-decreasing. N >= 2^30 is TC_ERR_UNSUPPORTED.
 *   Duplicate rows collapse; row order is irrelevant.
 * Blocks on a few small readbacks. *out is owned by the caller. */
tc_status tc_batch_from_ijk(const int32_t* d_ijk, const int64_t* h_offsets, int32_t grid_count,
                            const tc_allocator* allocator, void* stream, tc_grid_batch** out);

/* Builds a batch from float32 points (the points front-end beside the ijk
 * front-end; PR page, Measurements, follow-ups).
 *   d_xyz         float32[N][3] device, N = h_offsets[B]; may be NULL when N = 0.
 *   h_offsets     int64[B+1] host, as for tc_batch_from_ijk.
 *   h_voxel_size  float32[B][3] host, finite and > 0; h_origin float32[B][3] host, finite.
 *   mode          0: the voxel whose centre is nearest to the point, per axis
 *                    floor(x + 1/2) with x = (p - origin) / voxel_size computed in
 *                    float32 (a tie goes to the larger index);
 *                 1: the 8 voxels floor(x) + {0,1}^3 around the point.
 * Duplicates collapse. A point whose x is not finite is TC_ERR_INVALID_ARG, an
 * index outside int32 TC_ERR_OVERFLOW. More than 2^30 voxel rows (N, or 8N in
 * mode 1) is TC_ERR_UNSUPPORTED. Blocks on a few small readbacks. */
tc_status tc_batch_from_points(const float* d_xyz, const int64_t* h_offsets, int32_t grid_count,
                              const float* h_voxel_size, const float* h_origin, int32_t mode,
                              const tc_allocator* allocator, void* stream, tc_grid_batch** out);

/* One batched pass (or a chain of passes) over every member of `src`
 * (PR page section 1: emission, sorts, dedup, single readback, one allocation,
 * writers; section 2: box-dilate and pads; factors 4, 8 and k3s2 chain passes).
 *   op      a tc_op; factor as documented at tc_op.
 * `src` is borrowed and never modified. Blocks exactly once per pass, on one
 * readback; on return the host counts in tc_batch_info are valid and device
 * arrays are valid in stream order. Small batches (an output laid out by
 * capacities that fits in 32 MiB: at most 8 / 1 / 27 / 8 output leaves per
 * source leaf for refine / coarsen / dilate / pads, the tile and lower
 * candidates for the nodes, at most 1024 members and 262144 leaf slots) take
 * their one allocation after the node, marking and count launches, with no
 * readback before it, and read back all headers at the end (the voxel total is
 * then known too); their arrays sit at capacity offsets
 * inside the buffer and buffer_bytes is the capacity. Larger batches read the
 * per-grid node counts back first and allocate exactly.
 * Returns TC_ERR_OVERFLOW (and no batch) when any output voxel would leave int32,
 * TC_ERR_UNSUPPORTED for a non-power-of-two refine/coarsen factor. */
tc_status tc_build_batched_topology(const tc_grid_batch* src, int32_t op, int32_t factor,
                                    const tc_allocator* allocator, void* stream,
                                    tc_grid_batch** out);

/* Several generated targets of one source in one call (PR page section 1: the
 * per-iteration plan builds every target of a source; section 2: the box ops
 * and the k3s2 chain). Equivalent to n_ops calls of tc_build_batched_topology,
 * op h_ops[i] with factor h_factors[i] into out[i], on the same stream and
 * allocator, but the small-batch passes of consecutive ops are enqueued back to
 * back: each keeps its header readback pending, in a pinned host block of its
 * own, and the call waits once, at the end, for all of them (a chain's
 * intermediate passes still wait for their own counts).
 *   n_ops      >= 1; h_ops, h_factors int32[n_ops] host; out tc_grid_batch*[n_ops]
 *              host, every entry set (NULL on failure).
 * On return every out[i] is as tc_build_batched_topology leaves it. Validation
 * of every (op, factor) happens before any launch; an error in any op frees
 * every batch the call made and reports that op's status (its index in the
 * message when n_ops > 1). */
tc_status tc_build_batched_topology_many(const tc_grid_batch* src, int32_t n_ops, const int32_t* h_ops,
                                         const int32_t* h_factors, const tc_allocator* allocator,
                                         void* stream, tc_grid_batch** out);

/* Masked refine (PR page, test plan: masked refine): the voxels of `src` whose
 * keep flag is zero are dropped, the rest are refined by `factor` (2, 4 or 8),
 * as tc_build_batched_topology(TC_OP_REFINE) would refine the pruned batch.
 *   d_keep  device array of n_keep bytes, one per voxel of src in enumeration
 *           order (grid by grid, the order tc_enumerate_ijk writes); non-zero
 *           keeps the voxel. Read only; the caller keeps ownership.
 *   n_keep  must equal src's voxel total (tc_batch_voxel_total), else
 *           TC_ERR_INVALID_ARG; d_keep may be NULL only when it is 0.
 * Other arguments and the result as for tc_build_batched_topology. Blocks on the
 * voxel total (if not yet known), one flag check and the passes' readbacks. */
tc_status tc_build_masked_refine(const tc_grid_batch* src, const uint8_t* d_keep, int64_t n_keep,
                                 int32_t factor, const tc_allocator* allocator, void* stream,
                                 tc_grid_batch** out);

/* Counts (host) and device array pointers of a batch. Never blocks. */
tc_status tc_batch_get_info(const tc_grid_batch* batch, tc_batch_info* out);

/* Copies the B headers to host memory h_out (tc_grid_header[B]); this blocks on
 * `stream` (one small readback). Voxel counts and bboxes live only on the device
 * until this is called. */
tc_status tc_batch_read_headers(const tc_grid_batch* batch, tc_grid_header* h_out, void* stream);

/* Total voxel count of the batch (blocks like tc_batch_read_headers the first
 * time; cached afterwards). */
tc_status tc_batch_voxel_total(const tc_grid_batch* batch, int64_t* h_total, void* stream);

/* Writes the jagged voxel enumeration: d_ijk_out int32[V][3] device, V = voxel
 * total, grid after grid, each grid in canonical order (test plan: ijk.jdata);
 * member g's rows start at headers[g].voxel_begin. `capacity` is the row capacity
 * of d_ijk_out; fewer than V rows is TC_ERR_INVALID_ARG. Enqueues one kernel
 * (after a voxel-total readback the first time). */
tc_status tc_enumerate_ijk(const tc_grid_batch* batch, int32_t* d_ijk_out, int64_t capacity,
                           void* stream);

/* tc_enumerate_ijk of n batches in one launch (up to eight per launch, so a
 * group of small batches fills the device once instead of n times): batch j's
 * rows go to d_ijk_outs[j] (int32[V_j][3] device, capacities[j] >= V_j rows;
 * 16-byte aligned outputs take the vector stores). A NULL output is allowed for
 * a batch without voxels.
 *   n           >= 1; batches, d_ijk_outs, capacities: host arrays of n entries.
 * Every argument is checked before the launch. */
tc_status tc_enumerate_ijk_many(int32_t n, const tc_grid_batch* const* batches, int32_t* const* d_ijk_outs,
                                const int64_t* capacities, void* stream);

/* Kernel map of a convolution plan between two batches with the same member
 * count (issue page "Generated-topology grid construction dominates
 * per-iteration ConvolutionPlan cost", Measurements: a plan builds a k3 s1 map
 * on one topology and a k2s2 transposed-conv map; the layout is this library's).
 *   src, dst     source (input) and target (output) batches; read only.
 *   kernel_size  K in [1, 8]; offsets O_K = [-floor((K-1)/2), floor(K/2)] per
 *                axis, the same offset box as TC_OP_CONV_S1 / TC_OP_CONV_T_S1.
 *   stride       S in {1, 2} (others: TC_ERR_UNSUPPORTED).
 *   transposed   0: conv, target o reads source S*o + d;
 *                1: transposed conv, target o reads source (o - d)/S when S
 *                divides o - d in every component.
 *   d_out        device int32[V_dst][K^3]: row j = target voxel j in the order of
 *                tc_enumerate_ijk(dst), column k = offset d taken x-major,
 *                k = ((dx-lo)*K + (dy-lo))*K + (dz-lo) with lo = -floor((K-1)/2);
 *                the entry is the index (in the order of tc_enumerate_ijk(src))
 *                of the same member's source voxel, or -1. Owned by the caller.
 *   capacity     int32 entries available at d_out; fewer than V_dst * K^3 is
 *                TC_ERR_INVALID_ARG (d_out may be NULL only when that is 0).
 * Different member counts, K outside [1, 8] or S < 1 are TC_ERR_INVALID_ARG; a
 * source of more than INT32_MAX voxels is TC_ERR_UNSUPPORTED. Blocks on the two
 * voxel totals (if not yet known), then enqueues two kernels on `stream`. */
tc_status tc_build_kernel_map(const tc_grid_batch* src, const tc_grid_batch* dst, int32_t kernel_size,
                              int32_t stride, int32_t transposed, int32_t* d_out, int64_t capacity,
                              void* stream);

/* Kernel map with no allocation, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Arguments, output and errors as for tc_build_kernel_map;
 * it calls no hipMalloc, hipFree or other allocating routine, and reads the
 * voxel totals back into host stack memory when they are not yet known.
 * Scratch: a static device array of 64 MiB per GPU, loaded with the library
 * and held by every GPU it runs on until the process ends (its device address
 * is looked up on the first call on each device). The call needs
 *   256-byte aligned: 1 KiB per source upper node + 8 bytes per target leaf and
 *   window slot (8 to 64 slots, 27 for k3 s1) + 8 bytes per target leaf;
 * beyond 64 MiB it returns TC_ERR_UNSUPPORTED before any launch and writes
 * nothing. Every call on one GPU uses the same array, and no kernel relies on
 * what an earlier call left there: calls on one stream are ordered, but calls
 * that overlap on one GPU (other streams, other threads) race on it. */
tc_status tc_build_kernel_map_noalloc(const tc_grid_batch* src, const tc_grid_batch* dst, int32_t kernel_size,
                                      int32_t stride, int32_t transposed, int32_t* d_out, int64_t capacity,
                                      void* stream);

/* Cached device memory: every call takes its scratch arrays (and the buffers
 * of intermediate batches) from blocks cached process-wide per device, stream
 * and allocator, and keeps them for the next call with the same key (reuse is
 * ordered by that stream, so none is waited for). At most 24 idle blocks and
 * 8 GiB of idle bytes stay cached; beyond that the least recently used are
 * freed. tc_batch_free likewise keeps the buffer of a batch built without an
 * allocator (up to 64 buffers, 4 GiB) for the next batch on the same device
 * and stream. tc_scratch_release synchronizes the device, then frees every idle
 * scratch block (through its allocator's `free`, or to the device's pool) and
 * every cached batch buffer; later calls allocate again. Blocks in use by a
 * concurrent call are kept. Fails only with a HIP error. */
tc_status tc_scratch_release(void);

/* Releases the batch's device buffer (through the allocator it was created with,
 * stream-ordered on its creation stream) and the handle. NULL is ignored. */
void tc_batch_free(tc_grid_batch* batch);

/* Testing hook for the TC_ERR_INTERNAL path above: the next batch that the
 * calling thread builds (from ijk, from points, or as the output or an
 * intermediate of a pass) behaves as if its leaf-mask writers had flagged
 * `bits` (1 or 2; 0 cancels). That batch is written normally and its flags are
 * read back with its voxel total, so the error surfaces where a real one
 * would. Bits outside [0, 3] are TC_ERR_INVALID_ARG. */
tc_status tc_debug_inject_flags(int32_t bits);

/* Testing hook for the large-batch form of the box ops' leaf gather: while `on`
 * is 1, the calling thread's dilate and pad passes read their source arrays
 * through 64-bit addresses, as they do by themselves when a source array is
 * 2 GiB or more; 0 restores the default (32-bit buffer offsets below that
 * size). Results are the same either way. Values other than 0 and 1 are
 * TC_ERR_INVALID_ARG. */
tc_status tc_debug_wide_loads(int32_t on);

/* Kernel timing for measurement: while enabled, every launch of a kernel whose
 * name is in `kernel_names` (comma-separated __global__ function names, e.g.
 * "k_leaf_gather,k_enumerate"; "*" selects every kernel) is bracketed by HIP
 * events on the stream it is launched on. tc_profile_read() waits for those
 * events and returns the summed milliseconds and launch count of one kernel
 * since tc_profile_enable(). Not thread-safe against concurrent passes. */
tc_status tc_profile_enable(const char* kernel_names);
tc_status tc_profile_read(const char* kernel_name, double* h_total_ms, int64_t* h_launches);
tc_status tc_profile_disable(void);

#ifdef __cplusplus
}
#endif

#endif /* TOPO_H */
