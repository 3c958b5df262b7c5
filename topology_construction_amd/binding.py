"""Thin Python binding of the C ABI in include/topo.h (argument marshalling only).

Every step of the topology pass runs in the HIP library ``libtopo.so``; this
module only converts torch tensors to device pointers, passes torch's current
stream, supplies torch's caching allocator for the output buffers and wraps the
results as torch tensor views. It never computes topology itself and raises
when the library is missing.

Function names follow the C ABI (tc_batch_from_ijk, tc_build_batched_topology,
tc_enumerate_ijk, tc_batch_read_headers, ...).
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtopo.so")

TC_OK, TC_ERR_INVALID_ARG, TC_ERR_OVERFLOW, TC_ERR_ALLOC, TC_ERR_HIP, TC_ERR_UNSUPPORTED, TC_ERR_INTERNAL = range(7)
OPS = {"coarsen": 1, "refine": 2, "dilate": 3, "pad_neg": 4, "pad_pos": 5, "conv_t_k3s2": 6,
       "conv_s1": 7, "conv_t_s1": 8}

ABI_SYMBOLS = [
    "tc_abi_version", "tc_status_string", "tc_last_error", "tc_batch_from_ijk", "tc_batch_from_points",
    "tc_build_batched_topology", "tc_build_masked_refine", "tc_batch_get_info", "tc_batch_read_headers",
    "tc_batch_voxel_total", "tc_enumerate_ijk", "tc_build_kernel_map", "tc_scratch_release", "tc_batch_free",
    "tc_debug_inject_flags", "tc_build_kernel_map_noalloc", "tc_profile_enable", "tc_profile_read",
    "tc_profile_disable", "tc_build_batched_topology_many", "tc_enumerate_ijk_many", "tc_debug_wide_loads",
]

HEADER_DTYPE = np.dtype([
    ("grid_index", np.int32), ("grid_count", np.int32), ("upper_count", np.int32),
    ("lower_count", np.int32), ("leaf_count", np.int32), ("upper_begin", np.int32),
    ("lower_begin", np.int32), ("leaf_begin", np.int32), ("voxel_count", np.int64),
    ("voxel_begin", np.int64), ("bbox_min", np.int32, (3,)), ("bbox_max", np.int32, (3,)),
    ("reserved", np.int32, (2,)),
])
assert HEADER_DTYPE.itemsize == 80


class TopoError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


class tc_allocator(ctypes.Structure):
    _fields_ = [("alloc", ctypes.c_void_p), ("free", ctypes.c_void_p), ("ctx", ctypes.c_void_p)]


_P = ctypes.c_void_p


class tc_batch_info(ctypes.Structure):
    _fields_ = [
        ("grid_count", ctypes.c_int32), ("upper_count", ctypes.c_int32),
        ("lower_count", ctypes.c_int32), ("leaf_count", ctypes.c_int32),
        ("h_upper_counts", ctypes.POINTER(ctypes.c_int32)),
        ("h_lower_counts", ctypes.POINTER(ctypes.c_int32)),
        ("h_leaf_counts", ctypes.POINTER(ctypes.c_int32)),
        ("d_buffer", _P), ("buffer_bytes", ctypes.c_size_t),
        ("d_headers", _P), ("d_upper_origin", _P), ("d_upper_key", _P), ("d_upper_first", _P),
        ("d_upper_mask", _P), ("d_lower_origin", _P), ("d_lower_first", _P), ("d_lower_mask", _P),
        ("d_lower_prefix", _P), ("d_leaf_origin", _P), ("d_leaf_parent", _P), ("d_leaf_mask", _P),
        ("d_leaf_prefix", _P), ("d_leaf_offset", _P),
    ]


# field -> (info attribute, torch dtype name, row width, count attribute)
FIELDS = {
    "upper_origin": ("d_upper_origin", "int32", 4, "upper_count"),
    "upper_key": ("d_upper_key", "uint64", 1, "upper_count"),
    "upper_first": ("d_upper_first", "int32", 1, "upper_count"),
    "upper_mask": ("d_upper_mask", "uint64", 512, "upper_count"),
    "lower_origin": ("d_lower_origin", "int32", 4, "lower_count"),
    "lower_first": ("d_lower_first", "int32", 1, "lower_count"),
    "lower_mask": ("d_lower_mask", "uint64", 64, "lower_count"),
    "lower_prefix": ("d_lower_prefix", "uint16", 64, "lower_count"),
    "leaf_origin": ("d_leaf_origin", "int32", 4, "leaf_count"),
    "leaf_parent": ("d_leaf_parent", "int32", 1, "leaf_count"),
    "leaf_mask": ("d_leaf_mask", "uint64", 8, "leaf_count"),
    "leaf_prefix": ("d_leaf_prefix", "uint64", 1, "leaf_count"),
    "leaf_offset": ("d_leaf_offset", "int64", 1, "leaf_count"),
}

_ALLOC_FN = ctypes.CFUNCTYPE(ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p)
_FREE_FN = ctypes.CFUNCTYPE(None, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p)

_lock = threading.Lock()
_lib = None
_live_buffers: dict[int, object] = {}


def load_library(path: str = LIB_PATH):
    """Load libtopo.so and declare the C signatures. Raises if it is not built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with `python -m topology_construction_amd.build`")
        # torch first: its bundled HIP runtime (same SONAME) then serves this
        # library too, so streams and device pointers are shared by one runtime.
        import torch  # noqa: F401
        lib = ctypes.CDLL(path)
        i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        lib.tc_abi_version.restype = i32
        lib.tc_status_string.restype = ctypes.c_char_p
        lib.tc_status_string.argtypes = [ctypes.c_int]
        lib.tc_last_error.restype = ctypes.c_char_p
        lib.tc_batch_from_ijk.restype = ctypes.c_int
        lib.tc_batch_from_ijk.argtypes = [vp, vp, i32, vp, vp, ctypes.POINTER(vp)]
        lib.tc_build_batched_topology.restype = ctypes.c_int
        lib.tc_build_batched_topology.argtypes = [vp, i32, i32, vp, vp, ctypes.POINTER(vp)]
        lib.tc_build_batched_topology_many.restype = ctypes.c_int
        lib.tc_build_batched_topology_many.argtypes = [vp, i32, vp, vp, vp, vp, vp]
        lib.tc_enumerate_ijk_many.restype = ctypes.c_int
        lib.tc_enumerate_ijk_many.argtypes = [i32, vp, vp, vp, vp]
        lib.tc_build_masked_refine.restype = ctypes.c_int
        lib.tc_build_masked_refine.argtypes = [vp, vp, i64, i32, vp, vp, ctypes.POINTER(vp)]
        lib.tc_batch_get_info.restype = ctypes.c_int
        lib.tc_batch_get_info.argtypes = [vp, ctypes.POINTER(tc_batch_info)]
        lib.tc_batch_read_headers.restype = ctypes.c_int
        lib.tc_batch_read_headers.argtypes = [vp, vp, vp]
        lib.tc_batch_voxel_total.restype = ctypes.c_int
        lib.tc_batch_voxel_total.argtypes = [vp, ctypes.POINTER(i64), vp]
        lib.tc_enumerate_ijk.restype = ctypes.c_int
        lib.tc_enumerate_ijk.argtypes = [vp, vp, i64, vp]
        lib.tc_build_kernel_map.restype = ctypes.c_int
        lib.tc_build_kernel_map.argtypes = [vp, vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, i64, vp]
        lib.tc_build_kernel_map_noalloc.restype = ctypes.c_int
        lib.tc_build_kernel_map_noalloc.argtypes = [vp, vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, i64,
                                                    vp]
        lib.tc_batch_from_points.restype = ctypes.c_int
        lib.tc_batch_from_points.argtypes = [vp, vp, i32, vp, vp, i32, vp, vp, ctypes.POINTER(vp)]
        lib.tc_scratch_release.restype = ctypes.c_int
        lib.tc_scratch_release.argtypes = []
        lib.tc_batch_free.restype = None
        lib.tc_batch_free.argtypes = [vp]
        lib.tc_debug_inject_flags.restype = ctypes.c_int
        lib.tc_debug_inject_flags.argtypes = [i32]
        lib.tc_debug_wide_loads.restype = ctypes.c_int
        lib.tc_debug_wide_loads.argtypes = [i32]
        lib.tc_profile_enable.restype = ctypes.c_int
        lib.tc_profile_enable.argtypes = [ctypes.c_char_p]
        lib.tc_profile_read.restype = ctypes.c_int
        lib.tc_profile_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
        lib.tc_profile_disable.restype = ctypes.c_int
        if lib.tc_abi_version() != 1:
            raise ImportError("libtopo.so ABI version mismatch")
        _lib = lib
        return lib


def _check(status: int):
    if status != TC_OK:
        lib = load_library()
        raise TopoError(status, lib.tc_last_error().decode(errors="replace"))


def _current_raw_stream():
    """torch's current stream as a raw handle (None if torch cannot say cheaply)."""
    import torch
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    return int(raw(torch._C._cuda_getDevice())) if raw is not None else None


def _stream_handle(stream=None):
    import torch
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream)
    # the current stream's raw handle without building a Stream object per call
    raw = _current_raw_stream()
    if raw is not None:
        return ctypes.c_void_p(raw)
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


_stream_objs: dict = {}  # raw stream handle -> torch stream object wrapping it


def _torch_stream(handle: int):
    """A torch stream object for a raw hipStream_t handle (0: the null stream)."""
    import torch
    st = _stream_objs.get(handle)
    if st is None:
        st = torch.cuda.default_stream() if handle == 0 else torch.cuda.ExternalStream(handle)
        _stream_objs[handle] = st
    return st


def _empty_on(stream, shape, dtype):
    """torch.empty taken on `stream`, the stream the library writes the tensor on
    (the current stream when None), so torch's caching allocator orders its
    reuse after that stream's work."""
    import torch
    if stream is None:
        return torch.empty(shape, dtype=dtype, device="cuda")
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device="cuda")


def _torch_alloc(ctx, nbytes, stream):
    """Allocator callback: a uint8 tensor from torch's caching allocator, taken
    on the stream the library will use it on (so that torch hands the block to
    other work only in that stream's order once it is freed)."""
    try:
        import torch
        handle = int(stream or 0)
        n = max(int(nbytes), 1)
        cur = _current_raw_stream()
        if cur is not None and cur == handle:
            t = torch.empty(n, dtype=torch.uint8, device="cuda")
        else:
            with torch.cuda.stream(_torch_stream(handle)):
                t = torch.empty(n, dtype=torch.uint8, device="cuda")
        p = t.data_ptr()
        _live_buffers[p] = t
        return p
    except Exception:  # pragma: no cover - reported as TC_ERR_ALLOC by the library
        return None


def _torch_free(ctx, ptr, nbytes, stream):
    if _live_buffers is not None:  # None while the interpreter tears the module down
        _live_buffers.pop(int(ptr or 0), None)


_alloc_cb = _ALLOC_FN(_torch_alloc)
_free_cb = _FREE_FN(_torch_free)
TORCH_ALLOCATOR = tc_allocator(ctypes.cast(_alloc_cb, ctypes.c_void_p), ctypes.cast(_free_cb, ctypes.c_void_p), None)


class GridBatch:
    """Owner of a tc_grid_batch handle; tensor views share its device buffer."""

    def __init__(self, handle: ctypes.c_void_p, torch_owned: bool):
        self._lib = load_library()
        self.handle = handle
        self.torch_owned = torch_owned
        self._info_cache = None  # tc_batch_info, read on first use
        self._counts = None  # per-grid host counts, copied on first use
        self._total = None  # voxel total, once read
        self._buffer_cache = None

    @property
    def _info(self):
        if self._info_cache is None:
            info = tc_batch_info()
            _check(self._lib.tc_batch_get_info(self.handle, ctypes.byref(info)))
            self._info_cache = info
            if self.torch_owned:
                self._buffer_cache = _live_buffers.get(int(info.d_buffer or 0))
        return self._info_cache

    @property
    def _buffer(self):
        self._info  # noqa: B018 (reads the info, which finds the buffer)
        return self._buffer_cache

    @property
    def grid_count(self) -> int:
        return self._info.grid_count

    @property
    def upper_count(self) -> int:
        return self._info.upper_count

    @property
    def lower_count(self) -> int:
        return self._info.lower_count

    @property
    def leaf_count(self) -> int:
        return self._info.leaf_count

    def _grid_counts(self):
        if self._counts is None:
            B, info = self.grid_count, self._info
            self._counts = tuple(np.ctypeslib.as_array(p, (B,)).copy()
                                 for p in (info.h_upper_counts, info.h_lower_counts, info.h_leaf_counts))
        return self._counts

    @property
    def upper_counts(self) -> np.ndarray:
        return self._grid_counts()[0]

    @property
    def lower_counts(self) -> np.ndarray:
        return self._grid_counts()[1]

    @property
    def leaf_counts(self) -> np.ndarray:
        return self._grid_counts()[2]

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and getattr(self, "_lib", None) is not None:
            self._lib.tc_batch_free(h)
            self.handle = None

    def free(self):
        self.__del__()

    # -- device fields as torch tensors (views into the batch buffer) --------
    def field(self, name: str):
        import torch
        if self._buffer is None:
            raise RuntimeError("field views need a batch built with the torch allocator")
        attr, dt, width, count_attr = FIELDS[name]
        n = getattr(self, count_attr)
        start = int(getattr(self._info, attr) or 0) - int(self._info.d_buffer)
        dtype = getattr(torch, dt)
        nbytes = n * width * torch.empty(0, dtype=dtype).element_size()
        v = self._buffer[start:start + nbytes].view(dtype)
        return v.view(n, width) if width > 1 else v

    def fields(self) -> dict:
        return {k: self.field(k) for k in FIELDS}

    def headers(self, stream=None) -> np.ndarray:
        out = np.zeros(self.grid_count, dtype=HEADER_DTYPE)
        _check(self._lib.tc_batch_read_headers(self.handle, out.ctypes.data, _stream_handle(stream)))
        return out

    def voxel_total(self, stream=None) -> int:
        if self._total is None:  # the batch never changes: one read
            v = ctypes.c_int64()
            _check(self._lib.tc_batch_voxel_total(self.handle, ctypes.byref(v), _stream_handle(stream)))
            self._total = int(v.value)
        return self._total

    def ijk(self, stream=None):
        return tc_enumerate_ijk(self, stream=stream)


def tc_batch_from_ijk(ijk, offsets, stream=None, allocator: str = "torch") -> GridBatch:
    """Build a GridBatch from a device int32 [N, 3] tensor and int64 offsets [B+1]."""
    import torch
    lib = load_library()
    if not (isinstance(ijk, torch.Tensor) and ijk.is_cuda and ijk.dtype == torch.int32):
        raise TypeError("ijk must be a cuda int32 tensor")
    ijk = ijk.contiguous().view(-1, 3)
    off = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
    if off.ndim != 1 or off.shape[0] < 2 or int(off[-1]) != ijk.shape[0]:
        raise ValueError("offsets must be [B+1] with offsets[-1] == number of rows")
    alloc = ctypes.byref(TORCH_ALLOCATOR) if allocator == "torch" else None
    h = ctypes.c_void_p()
    _check(lib.tc_batch_from_ijk(ctypes.c_void_p(ijk.data_ptr() if ijk.numel() else 0), off.ctypes.data,
                                 off.shape[0] - 1, alloc, _stream_handle(stream), ctypes.byref(h)))
    return GridBatch(h, allocator == "torch")


def tc_batch_from_points(points, offsets, voxel_size, origin, mode: int = 0, stream=None,
                         allocator: str = "torch") -> GridBatch:
    """Build a GridBatch from a device float32 [N, 3] tensor of points, int64
    offsets [B+1] and per-member voxel sizes / origins ([B, 3], host). mode 0:
    the voxel of the nearest centre; mode 1: the 8 voxels around each point."""
    import torch
    lib = load_library()
    if not (isinstance(points, torch.Tensor) and points.is_cuda and points.dtype == torch.float32):
        raise TypeError("points must be a cuda float32 tensor")
    points = points.contiguous().view(-1, 3)
    off = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
    if off.ndim != 1 or off.shape[0] < 2 or int(off[-1]) != points.shape[0]:
        raise ValueError("offsets must be [B+1] with offsets[-1] == number of points")
    vs = np.ascontiguousarray(np.asarray(voxel_size, dtype=np.float32).reshape(-1, 3))
    org = np.ascontiguousarray(np.asarray(origin, dtype=np.float32).reshape(-1, 3))
    if vs.shape[0] != off.shape[0] - 1 or org.shape[0] != off.shape[0] - 1:
        raise ValueError("voxel_size and origin must be [B, 3]")
    alloc = ctypes.byref(TORCH_ALLOCATOR) if allocator == "torch" else None
    h = ctypes.c_void_p()
    _check(lib.tc_batch_from_points(ctypes.c_void_p(points.data_ptr() if points.numel() else 0), off.ctypes.data,
                                    off.shape[0] - 1, vs.ctypes.data, org.ctypes.data, int(mode), alloc,
                                    _stream_handle(stream), ctypes.byref(h)))
    return GridBatch(h, allocator == "torch")


def tc_build_batched_topology(src: GridBatch, op, factor: int, stream=None, allocator: str = "torch") -> GridBatch:
    """Run the batched topology pass(es) `op` (name or tc_op id) with `factor`."""
    lib = load_library()
    op_id = OPS[op] if isinstance(op, str) else int(op)
    alloc = ctypes.byref(TORCH_ALLOCATOR) if allocator == "torch" else None
    h = ctypes.c_void_p()
    _check(lib.tc_build_batched_topology(src.handle, op_id, int(factor), alloc, _stream_handle(stream),
                                         ctypes.byref(h)))
    return GridBatch(h, allocator == "torch")


def tc_build_batched_topology_many(src: GridBatch, ops, stream=None, allocator: str = "torch") -> list:
    """Several targets of one source in one call: `ops` is a sequence of
    (op, factor) pairs (op a name or tc_op id); returns one GridBatch per pair."""
    lib = load_library()
    ops = list(ops)
    n = len(ops)
    if n < 1:
        raise ValueError("ops is empty")
    op_ids = (ctypes.c_int32 * n)(*[OPS[o] if isinstance(o, str) else int(o) for o, _ in ops])
    factors = (ctypes.c_int32 * n)(*[int(f) for _, f in ops])
    handles = (ctypes.c_void_p * n)()
    alloc = ctypes.byref(TORCH_ALLOCATOR) if allocator == "torch" else None
    _check(lib.tc_build_batched_topology_many(src.handle, n, op_ids, factors, alloc, _stream_handle(stream), handles))
    out = []
    try:
        for i in range(n):
            out.append(GridBatch(ctypes.c_void_p(handles[i]), allocator == "torch"))
    except BaseException:
        for j in range(len(out) + 1, n):  # handles not wrapped yet (the failed one frees itself)
            lib.tc_batch_free(ctypes.c_void_p(handles[j]))
        raise
    return out


def tc_build_masked_refine(src: GridBatch, keep, factor: int, stream=None, allocator: str = "torch") -> GridBatch:
    """Masked refine: `keep` is a device uint8 (or bool) tensor, one flag per voxel
    of `src` in enumeration order; kept voxels are refined by `factor`."""
    import torch
    lib = load_library()
    if keep.device.type != "cuda" or keep.dim() != 1:
        raise ValueError("keep must be a 1-D device tensor")
    keep = keep.to(torch.uint8).contiguous()
    alloc = ctypes.byref(TORCH_ALLOCATOR) if allocator == "torch" else None
    h = ctypes.c_void_p()
    _check(lib.tc_build_masked_refine(src.handle, keep.data_ptr() if keep.numel() else None, int(keep.numel()),
                                      int(factor), alloc, _stream_handle(stream), ctypes.byref(h)))
    return GridBatch(h, allocator == "torch")


def tc_enumerate_ijk(batch: GridBatch, out=None, stream=None):
    """Jagged voxel enumeration int32 [V, 3] (grid after grid, canonical order),
    written on `stream` (torch's current stream when None): a reader on another
    stream synchronizes with it first."""
    import torch
    lib = load_library()
    total = batch.voxel_total(stream)
    if out is None:
        out = _empty_on(stream, (total, 3), torch.int32)
    cap = out.shape[0] if out.dim() == 2 else out.numel() // 3
    _check(lib.tc_enumerate_ijk(batch.handle, ctypes.c_void_p(out.data_ptr() if out.numel() else 0), int(cap),
                                _stream_handle(stream)))
    return out[:total]


def tc_enumerate_ijk_many(batches, stream=None) -> list:
    """Jagged voxel enumerations of several batches in one launch: one int32
    [V_j, 3] view per batch into one allocation (each view starting on a
    16-byte boundary)."""
    import torch
    lib = load_library()
    batches = list(batches)
    n = len(batches)
    if n < 1:
        raise ValueError("batches is empty")
    totals = [b.voxel_total(stream) for b in batches]
    starts, at = [], 0
    for t in totals:
        starts.append(at)
        at += (t + 3) // 4 * 4  # rows of 12 bytes: a multiple of 4 rows keeps 16-byte alignment
    buf = _empty_on(stream, (max(at, 1), 3), torch.int32)
    base = buf.data_ptr()
    outs = (ctypes.c_void_p * n)(*[base + 12 * a if t else 0 for a, t in zip(starts, totals)])
    caps = (ctypes.c_int64 * n)(*totals)
    hs = (ctypes.c_void_p * n)(*[b.handle.value if isinstance(b.handle, ctypes.c_void_p) else b.handle
                                 for b in batches])
    _check(lib.tc_enumerate_ijk_many(n, hs, outs, caps, _stream_handle(stream)))
    return [buf[a:a + t] for a, t in zip(starts, totals)]


def tc_build_kernel_map(src: GridBatch, dst: GridBatch, kernel_size: int, stride: int, transposed: bool,
                        out=None, stream=None):
    """Kernel map int32 [V_dst, K^3]: for target voxel j and x-major offset k, the
    index of the source voxel it reads (S*o + d, or (o - d)/S transposed), or -1."""
    import torch
    lib = load_library()
    kk = int(kernel_size) ** 3
    rows = dst.voxel_total(stream)
    if out is None:
        out = _empty_on(stream, (rows, kk), torch.int32)
    _check(lib.tc_build_kernel_map(src.handle, dst.handle, int(kernel_size), int(stride), int(bool(transposed)),
                                   ctypes.c_void_p(out.data_ptr() if out.numel() else 0), int(out.numel()),
                                   _stream_handle(stream)))
    return out.view(-1)[:rows * kk].view(rows, kk)


def tc_build_kernel_map_noalloc(src: GridBatch, dst: GridBatch, kernel_size: int, stride: int, transposed: bool,
                                out, stream=None):
    """As tc_build_kernel_map into a caller-allocated `out`, with the library's
    static scratch (no device allocation by the library)."""
    kk = int(kernel_size) ** 3
    rows = dst.voxel_total(stream)
    _check(load_library().tc_build_kernel_map_noalloc(
        src.handle, dst.handle, int(kernel_size), int(stride), int(bool(transposed)),
        ctypes.c_void_p(out.data_ptr() if out.numel() else 0), int(out.numel()), _stream_handle(stream)))
    return out.view(-1)[:rows * kk].view(rows, kk)


def tc_scratch_release():
    """Free every idle cached scratch block and cached batch buffer."""
    _check(load_library().tc_scratch_release())


def tc_batch_read_headers(batch: GridBatch, stream=None) -> np.ndarray:
    return batch.headers(stream)


def tc_debug_wide_loads(on: bool):
    """Testing: this thread's box-op passes read their sources through 64-bit
    addresses (the form for source arrays of 2 GiB or more) while `on`."""
    _check(load_library().tc_debug_wide_loads(1 if on else 0))


def tc_debug_inject_flags(bits: int):
    """Testing: the next batch built on this thread reports a failed device
    consistency check of its writers (TC_ERR_INTERNAL at its first blocking read)."""
    _check(load_library().tc_debug_inject_flags(int(bits)))


def tc_profile_enable(kernel_names: str):
    """Time launches of the named kernels (comma-separated, or "*") with HIP events."""
    _check(load_library().tc_profile_enable(kernel_names.encode()))


def tc_profile_read(kernel_name: str):
    """(total ms, launches) of one kernel since tc_profile_enable."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(load_library().tc_profile_read(kernel_name.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return float(ms.value), int(n.value)


def tc_profile_disable():
    _check(load_library().tc_profile_disable())
