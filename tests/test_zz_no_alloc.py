"""The no-allocation kernel map (tc_build_kernel_map_noalloc) against the
allocating one (tc_build_kernel_map), through the C ABI: two calls in a row,
the second on a smaller input, each equal to the allocating entry point's
table element by element; a call whose scratch would exceed the static array
is refused before it writes anything."""
import ctypes

import numpy as np
import pytest

from topology_construction_amd import binding, synth

pytestmark = pytest.mark.gpu


def _batch(ijk, off):
    import torch
    return binding.tc_batch_from_ijk(torch.from_numpy(np.ascontiguousarray(ijk, dtype=np.int32)).cuda(), off)


def _noalloc(lib, src, dst, k, s, t, out):
    return lib.tc_build_kernel_map_noalloc(src.handle, dst.handle, k, s, t, ctypes.c_void_p(out.data_ptr()),
                                           out.numel(), None)


def test_noalloc_kernel_map_matches_allocating_entry_point():
    import torch
    lib = binding.load_library()
    big_ijk, big_off = synth.make_config(2)     # 16 res-64 shells
    small_ijk, small_off = synth.make_config(1)  # 2 res-16 shells
    cases = []
    for ijk, off in [(big_ijk, big_off), (small_ijk, small_off)]:
        src = _batch(ijk, off)
        fine = binding.tc_build_batched_topology(src, "refine", 2)
        cases.append((src, src, 3, 1, 0))
        cases.append((src, fine, 2, 2, 1))
    # two calls in a row per map kind, the second on the smaller batch
    for (src, dst, k, s, t) in [cases[0], cases[2], cases[1], cases[3]]:
        rows = dst.voxel_total()
        ref = binding.tc_build_kernel_map(src, dst, k, s, bool(t))
        out = torch.full((rows, k ** 3), -7, dtype=torch.int32, device="cuda")
        st = _noalloc(lib, src, dst, k, s, t, out)
        assert st == binding.TC_OK, lib.tc_last_error()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"k={k} s={s} t={t} rows={rows}"


def test_noalloc_refuses_scratch_beyond_the_static_array():
    import torch
    lib = binding.load_library()
    # 70^3 isolated voxels, one per leaf: a k3 s1 map needs 27 window slots per
    # target leaf, 8 bytes each, i.e. ~74 MB of scratch (> 64 MiB)
    g = np.arange(70, dtype=np.int32) * 8
    ijk = np.stack(np.meshgrid(g, g, g, indexing="ij"), -1).reshape(-1, 3)
    src = _batch(ijk, np.array([0, ijk.shape[0]], np.int64))
    assert src.leaf_count == 70 ** 3
    out = torch.full((ijk.shape[0], 27), -7, dtype=torch.int32, device="cuda")
    st = _noalloc(lib, src, src, 3, 1, 0, out)
    assert st == binding.TC_ERR_UNSUPPORTED
    assert b"scratch" in lib.tc_last_error()
    torch.cuda.synchronize()
    assert bool((out == -7).all()), "a refused call wrote output"
    # the allocating entry point takes the same map
    ref = binding.tc_build_kernel_map(src, src, 3, 1, False)
    assert bool((ref[:, 13] == torch.arange(ijk.shape[0], device="cuda", dtype=torch.int32)).all())
    # and the static array still serves a call that fits afterwards
    small_ijk, small_off = synth.make_config(1)
    s2 = _batch(small_ijk, small_off)
    o2 = torch.empty((s2.voxel_total(), 27), dtype=torch.int32, device="cuda")
    assert _noalloc(lib, s2, s2, 3, 1, 0, o2) == binding.TC_OK
    torch.cuda.synchronize()
    assert torch.equal(o2, binding.tc_build_kernel_map(s2, s2, 3, 1, False))
