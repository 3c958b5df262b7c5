"""C-ABI checks that need no GPU: the library loads, exports every function that
include/topo.h declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

from topology_construction_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "topo.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(tc_[a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def test_header_declares_the_binding_symbols():
    assert _declared_functions() == sorted(binding.ABI_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert lib.tc_abi_version() == 1


def test_library_has_gfx950_code_object():
    data = open(binding.LIB_PATH, "rb").read()
    assert b"gfx950" in data


def test_status_strings(lib):
    assert lib.tc_status_string(0) == b"ok"
    assert lib.tc_status_string(2) == b"int32 coordinate overflow"
    assert lib.tc_status_string(99) == b"unknown status"


def test_from_ijk_rejects_bad_arguments_on_host(lib):
    out = ctypes.c_void_p(123)
    off = (ctypes.c_int64 * 3)(0, 2, 1)  # decreasing
    st = lib.tc_batch_from_ijk(None, off, 2, None, None, ctypes.byref(out))
    assert st == binding.TC_ERR_INVALID_ARG and out.value is None
    assert b"non-decreasing" in lib.tc_last_error()
    off0 = (ctypes.c_int64 * 1)(0)
    assert lib.tc_batch_from_ijk(None, off0, 0, None, None, ctypes.byref(out)) == binding.TC_ERR_INVALID_ARG
    off1 = (ctypes.c_int64 * 2)(1, 2)
    assert lib.tc_batch_from_ijk(None, off1, 1, None, None, ctypes.byref(out)) == binding.TC_ERR_INVALID_ARG
    off2 = (ctypes.c_int64 * 2)(0, 5)
    assert lib.tc_batch_from_ijk(None, off2, 1, None, None, ctypes.byref(out)) == binding.TC_ERR_INVALID_ARG
    assert b"d_ijk" in lib.tc_last_error()
    off3 = (ctypes.c_int64 * 2)(0, 1 << 31)
    assert lib.tc_batch_from_ijk(ctypes.c_void_p(8), off3, 1, None, None, ctypes.byref(out)) == binding.TC_ERR_UNSUPPORTED
    assert lib.tc_batch_from_ijk(None, off0, 1, None, None, None) == binding.TC_ERR_INVALID_ARG
    bad_alloc = binding.tc_allocator(None, None, None)
    off4 = (ctypes.c_int64 * 2)(0, 0)
    assert lib.tc_batch_from_ijk(None, off4, 1, ctypes.byref(bad_alloc), None, ctypes.byref(out)) == binding.TC_ERR_INVALID_ARG


def test_build_rejects_bad_arguments_on_host(lib):
    out = ctypes.c_void_p(123)
    assert lib.tc_build_batched_topology(None, 2, 2, None, None, ctypes.byref(out)) == binding.TC_ERR_INVALID_ARG
    assert out.value is None
    assert b"src" in lib.tc_last_error()
    assert lib.tc_build_batched_topology(None, 2, 2, None, None, None) == binding.TC_ERR_INVALID_ARG


def test_build_many_rejects_bad_arguments_on_host(lib):
    ops = (ctypes.c_int32 * 2)(binding.OPS["refine"], binding.OPS["dilate"])
    facs = (ctypes.c_int32 * 2)(2, 1)
    outs = (ctypes.c_void_p * 2)(123, 456)
    assert lib.tc_build_batched_topology_many(None, 2, ops, facs, None, None, outs) == binding.TC_ERR_INVALID_ARG
    assert outs[0] is None and outs[1] is None
    assert b"src" in lib.tc_last_error()
    assert lib.tc_build_batched_topology_many(None, 0, ops, facs, None, None, outs) == binding.TC_ERR_INVALID_ARG
    assert b"n_ops" in lib.tc_last_error()
    assert lib.tc_build_batched_topology_many(None, 2, None, facs, None, None, outs) == binding.TC_ERR_INVALID_ARG
    assert lib.tc_build_batched_topology_many(None, 2, ops, facs, None, None, None) == binding.TC_ERR_INVALID_ARG


def test_enumerate_many_rejects_bad_arguments_on_host(lib):
    outs = (ctypes.c_void_p * 2)()
    caps = (ctypes.c_int64 * 2)(0, 0)
    hs = (ctypes.c_void_p * 2)()
    assert lib.tc_enumerate_ijk_many(0, hs, outs, caps, None) == binding.TC_ERR_INVALID_ARG
    assert lib.tc_enumerate_ijk_many(2, None, outs, caps, None) == binding.TC_ERR_INVALID_ARG
    assert lib.tc_enumerate_ijk_many(2, hs, outs, caps, None) == binding.TC_ERR_INVALID_ARG
    assert b"batch 0 is NULL" in lib.tc_last_error()


def test_null_handles_are_rejected(lib):
    info = binding.tc_batch_info()
    assert lib.tc_batch_get_info(None, ctypes.byref(info)) == binding.TC_ERR_INVALID_ARG
    assert lib.tc_batch_read_headers(None, None, None) == binding.TC_ERR_INVALID_ARG
    v = ctypes.c_int64()
    assert lib.tc_batch_voxel_total(None, ctypes.byref(v), None) == binding.TC_ERR_INVALID_ARG
    assert lib.tc_enumerate_ijk(None, None, 0, None) == binding.TC_ERR_INVALID_ARG
    lib.tc_batch_free(None)  # no-op


def test_profiling_state_machine_without_launches(lib):
    assert lib.tc_profile_enable(None) == binding.TC_ERR_INVALID_ARG
    assert lib.tc_profile_enable(b"k_leaf_gather, k_enumerate") == 0
    ms, n = ctypes.c_double(), ctypes.c_int64()
    assert lib.tc_profile_read(b"k_enumerate", ctypes.byref(ms), ctypes.byref(n)) == 0
    assert lib.tc_profile_read(None, ctypes.byref(ms), ctypes.byref(n)) == binding.TC_ERR_INVALID_ARG
    assert n.value == 0 and ms.value == 0.0
    assert lib.tc_profile_disable() == 0


def test_header_struct_layout_matches_binding():
    assert binding.HEADER_DTYPE.itemsize == 80
    assert binding.HEADER_DTYPE.fields["voxel_count"][1] == 32
    assert binding.HEADER_DTYPE.fields["bbox_min"][1] == 48


def test_no_kernel_uses_scratch_memory(tmp_path):
    """Every kernel keeps its arrays in registers or LDS: a runtime index into a
    register array (or a spill) would put it in scratch memory, which lives in HBM
    and once cost one gather kernel twice its time. Compiles the device code of
    every source for gfx950 to assembly and reads each kernel's private segment."""
    import subprocess
    from topology_construction_amd import build
    csrc = build.CSRC
    bad = []
    for src in build.SOURCES:
        out = tmp_path / (src + ".s")
        subprocess.check_call([build.HIPCC, f"--offload-arch={build.ARCH}", "-O3", "-std=c++17",
                               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                               "--cuda-device-only", "-S", os.path.join(csrc, src), "-o", str(out)],
                              stderr=subprocess.DEVNULL)
        text = out.read_text()
        for m in re.finditer(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", text, flags=re.S):
            seg = re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", m.group(2))
            if seg and int(seg.group(1)) != 0:
                bad.append((src, m.group(1), int(seg.group(1))))
    assert not bad, bad


def test_debug_inject_flags_validates_on_host(lib):
    assert lib.tc_debug_inject_flags(7) == binding.TC_ERR_INVALID_ARG
    assert lib.tc_debug_inject_flags(-1) == binding.TC_ERR_INVALID_ARG
    assert b"bits" in lib.tc_last_error()
    assert lib.tc_debug_inject_flags(0) == binding.TC_OK  # cancels (nothing armed here)


def test_debug_wide_loads_validates_on_host(lib):
    assert lib.tc_debug_wide_loads(2) == binding.TC_ERR_INVALID_ARG
    assert lib.tc_debug_wide_loads(-1) == binding.TC_ERR_INVALID_ARG
    assert b"on must be" in lib.tc_last_error()
    assert lib.tc_debug_wide_loads(1) == binding.TC_OK
    assert lib.tc_debug_wide_loads(0) == binding.TC_OK
