"""CPU oracle for batched generated-topology construction (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package. The HIP library never links, loads or calls it,
and it shares no code with the library. The arithmetic lives in
``oracle/oracle.cpp`` (plain C++, compiled with g++); this module compiles it on
demand and marshals numpy arrays in and out.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.cpp")
LIB = os.path.join(HERE, "liboracle.so")

# Op ids, as documented in oracle.cpp.
IDENTITY, COARSEN, REFINE, DILATE, PAD_NEG, PAD_POS, CONV_T_K3S2, CONV_S1, CONV_T_S1 = range(9)
OP_IDS = {
    "identity": IDENTITY, "coarsen": COARSEN, "refine": REFINE, "dilate": DILATE,
    "pad_neg": PAD_NEG, "pad_pos": PAD_POS, "conv_t_k3s2": CONV_T_K3S2,
    "conv_s1": CONV_S1, "conv_t_s1": CONV_T_S1,
}

OK, INVALID, OVERFLOW, NOMEM = 0, 1, 2, 3

# (field id, dtype, row width)
FIELDS = {
    "headers": (0, np.int64, 16),
    "upper_origin": (1, np.int32, 4),
    "upper_key": (2, np.uint64, 1),
    "upper_first": (3, np.int32, 1),
    "upper_mask": (4, np.uint64, 512),
    "lower_origin": (5, np.int32, 4),
    "lower_first": (6, np.int32, 1),
    "lower_mask": (7, np.uint64, 64),
    "lower_prefix": (8, np.uint16, 64),
    "leaf_origin": (9, np.int32, 4),
    "leaf_parent": (10, np.int32, 1),
    "leaf_mask": (11, np.uint64, 8),
    "leaf_prefix": (12, np.uint64, 1),
    "leaf_offset": (13, np.int64, 1),
    "ijk": (14, np.int32, 3),
}

HEADER_COLUMNS = [
    "grid_index", "grid_count", "upper_count", "lower_count", "leaf_count",
    "upper_begin", "lower_begin", "leaf_begin", "voxel_count", "voxel_begin",
    "bbox_min_x", "bbox_min_y", "bbox_min_z", "bbox_max_x", "bbox_max_y", "bbox_max_z",
]

_lock = threading.Lock()
_lib = None


class OracleError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"oracle status {status}")
        self.status = status


def build(force: bool = False) -> str:
    """Compile oracle.cpp into liboracle.so with g++ (no GPU code involved)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(
            ["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-o", tmp, SRC])
        os.replace(tmp, LIB)
    return LIB


def bind(path: str):
    """Load a compiled oracle library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    lib.oracle_build.restype = ctypes.c_int
    lib.oracle_build.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_int32,
                                 ctypes.POINTER(ctypes.c_void_p)]
    lib.oracle_build_threaded.restype = ctypes.c_int
    lib.oracle_build_threaded.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.POINTER(ctypes.c_void_p)]
    lib.oracle_build_masked_refine.restype = ctypes.c_int
    lib.oracle_build_masked_refine.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                               ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(ctypes.c_void_p)]
    lib.oracle_kernel_map.restype = ctypes.c_int
    lib.oracle_kernel_map.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_int32, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.oracle_size.restype = ctypes.c_int64
    lib.oracle_size.argtypes = [ctypes.c_void_p, ctypes.c_int]
    lib.oracle_copy.restype = ctypes.c_int
    lib.oracle_copy.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.oracle_free.restype = None
    lib.oracle_free.argtypes = [ctypes.c_void_p]
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            _lib = bind(LIB)
    return _lib


def _collect(lib, handle, fields):
    try:
        out = {}
        for name in (fields or FIELDS.keys()):
            fid, dt, width = FIELDS[name]
            n = lib.oracle_size(handle, fid)
            arr = np.empty(n, dtype=dt)
            if n:
                lib.oracle_copy(handle, fid, arr.ctypes.data)
            out[name] = arr.reshape(-1, width) if width > 1 else arr
        return out
    finally:
        lib.oracle_free(handle)


def run_masked_refine(factor: int, ijk: np.ndarray, offsets: np.ndarray, keep: np.ndarray, fields=None,
                      lib=None) -> dict:
    """Masked refine: keep (one byte per voxel, in the canonical enumeration order
    of the batch built from ijk) prunes voxels, the rest are refined by factor."""
    lib = lib or _load()
    ijk = np.ascontiguousarray(np.asarray(ijk, dtype=np.int32).reshape(-1, 3))
    offsets = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
    keep = np.ascontiguousarray(np.asarray(keep, dtype=np.uint8).reshape(-1))
    handle = ctypes.c_void_p()
    st = lib.oracle_build_masked_refine(int(factor), ijk.ctypes.data if ijk.size else None, offsets.ctypes.data,
                                        int(offsets.shape[0]) - 1, keep.ctypes.data if keep.size else None,
                                        int(keep.shape[0]), ctypes.byref(handle))
    if st != OK:
        raise OracleError(st)
    return _collect(lib, handle, fields)


def run(op, factor: int, ijk: np.ndarray, offsets: np.ndarray, fields=None, lib=None) -> dict:
    """Run the oracle; returns {field: numpy array} (rows reshaped to the field's width).

    Raises OracleError(status) for invalid arguments (1) or int32 overflow (2).
    ``lib`` selects another compiled oracle (used to check that planted mistakes
    are caught by the pins).
    """
    lib = lib or _load()
    if isinstance(op, str):
        op = OP_IDS[op]
    ijk = np.ascontiguousarray(np.asarray(ijk, dtype=np.int32).reshape(-1, 3))
    offsets = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
    B = int(offsets.shape[0]) - 1
    handle = ctypes.c_void_p()
    st = lib.oracle_build(int(op), int(factor),
                          ijk.ctypes.data if ijk.size else None,
                          offsets.ctypes.data, B, ctypes.byref(handle))
    if st != OK:
        raise OracleError(st)
    return _collect(lib, handle, fields)


def run_threaded(op, factor: int, ijk: np.ndarray, offsets: np.ndarray, threads: int = 0, fields=None,
                 lib=None) -> dict:
    """As run(), with the members built in parallel by `threads` host threads
    (0: host_threads()), each as a batch of one, and concatenated in member
    order (oracle_build_threaded). The per-member arithmetic is run()'s."""
    lib = lib or _load()
    threads = int(threads) if threads else host_threads()
    if isinstance(op, str):
        op = OP_IDS[op]
    ijk = np.ascontiguousarray(np.asarray(ijk, dtype=np.int32).reshape(-1, 3))
    offsets = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
    handle = ctypes.c_void_p()
    st = lib.oracle_build_threaded(int(op), int(factor), ijk.ctypes.data if ijk.size else None,
                                   offsets.ctypes.data, int(offsets.shape[0]) - 1, int(threads),
                                   ctypes.byref(handle))
    if st != OK:
        raise OracleError(st)
    return _collect(lib, handle, fields)


def host_threads() -> int:
    """Host threads for the threaded driver: OMP_NUM_THREADS when set (a machine
    that shares its cores states this process's share there), else the cores
    this process may run on."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except (AttributeError, OSError):  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def member_offsets(result: dict) -> np.ndarray:
    """Member row offsets of a result's enumeration, from its headers."""
    h = result["headers"]
    return np.concatenate([h[:, 9], [h[-1, 9] + h[-1, 8]]]).astype(np.int64)


def kernel_map_rows(src_ijk, src_off, dst_ijk, dst_off, kernel: int, stride: int, transposed: bool,
                    lib=None) -> np.ndarray:
    """Kernel map (int32 [V_dst, K^3], -1 where no source voxel) between two batches
    given as canonical enumerations: ijk rows and member row offsets."""
    lib = lib or _load()
    src_ijk = np.ascontiguousarray(np.asarray(src_ijk, dtype=np.int32).reshape(-1, 3))
    dst_ijk = np.ascontiguousarray(np.asarray(dst_ijk, dtype=np.int32).reshape(-1, 3))
    src_off = np.ascontiguousarray(np.asarray(src_off, dtype=np.int64))
    dst_off = np.ascontiguousarray(np.asarray(dst_off, dtype=np.int64))
    if src_off.shape != dst_off.shape:
        raise ValueError("source and target member counts differ")
    kk = int(kernel) ** 3
    out = np.empty((dst_ijk.shape[0], kk), dtype=np.int32)
    st = lib.oracle_kernel_map(src_ijk.ctypes.data if src_ijk.size else None, src_off.ctypes.data,
                               dst_ijk.ctypes.data if dst_ijk.size else None, dst_off.ctypes.data,
                               int(src_off.shape[0]) - 1, int(kernel), int(stride), int(bool(transposed)),
                               out.ctypes.data if out.size else None)
    if st != OK:
        raise OracleError(st)
    return out


def kernel_map(src: dict, dst: dict, kernel: int, stride: int, transposed: bool, **kw) -> np.ndarray:
    """Kernel map between two oracle results (each holding "ijk" and "headers")."""
    return kernel_map_rows(src["ijk"], member_offsets(src), dst["ijk"], member_offsets(dst), kernel, stride,
                           transposed, **kw)


# ---------------------------------------------------------------- points front-end
# The issue/PR pages list from_points beside from_ijk as a front-end that feeds
# the same batched back-end (PR page, Measurements, follow-ups). Reading (the
# pages give no formula): member g's point p lies in index space at
# x = (p - origin_g) / voxel_size_g, computed in float32 as the kernels do;
#   mode 0 (voxel of the point): the voxel whose centre is nearest, floor(x + 1/2)
#          per axis (a tie goes to the larger index);
#   mode 1 (nearest voxels):      the 2^3 voxels around it, floor(x) + {0, 1}^3.
# Duplicates collapse as in from_ijk. A non-finite x is an invalid argument, an
# index outside int32 an overflow.
def points_to_ijk(points, offsets, voxel_size, origin, mode: int):
    """int32 ijk rows and member offsets for the points front-end (float32 arithmetic)."""
    pts = np.asarray(points, dtype=np.float32).reshape(-1, 3)
    off = np.asarray(offsets, dtype=np.int64)
    vs = np.asarray(voxel_size, dtype=np.float32).reshape(-1, 3)
    org = np.asarray(origin, dtype=np.float32).reshape(-1, 3)
    B = off.shape[0] - 1
    if vs.shape[0] != B or org.shape[0] != B or mode not in (0, 1):
        raise OracleError(INVALID)
    if not (np.isfinite(vs).all() and (vs > 0).all() and np.isfinite(org).all()):
        raise OracleError(INVALID)
    g = np.repeat(np.arange(B), np.diff(off))
    with np.errstate(all="ignore"):
        x = (pts - org[g]) / vs[g]  # float32 subtract, then float32 divide
        if not np.isfinite(x).all():
            raise OracleError(INVALID)
        base = np.floor(x + np.float32(0.5)) if mode == 0 else np.floor(x)
    hi = base.max(initial=0) + (1 if mode == 1 else 0)
    if base.size and (base.min() < -2.0 ** 31 or hi > 2.0 ** 31 - 1):
        raise OracleError(OVERFLOW)
    base = base.astype(np.int64)
    if mode == 0:
        return base.astype(np.int32), off.copy()
    corners = np.array([[a, b, c] for a in (0, 1) for b in (0, 1) for c in (0, 1)], dtype=np.int64)
    rows = (base[:, None, :] + corners[None, :, :]).reshape(-1, 3)
    return rows.astype(np.int32), off * 8


def run_points(points, offsets, voxel_size, origin, mode: int, fields=None, lib=None) -> dict:
    """Oracle batch built from points: points_to_ijk, then the ijk front-end."""
    ijk, off = points_to_ijk(points, offsets, voxel_size, origin, mode)
    return run(IDENTITY, 1, ijk, off, fields=fields, lib=lib)
