"""HIP path vs oracle, element by element, through the C ABI.

Every array the library exposes (headers, upper/lower/leaf records, masks,
prefix words, offsets, the jagged ijk enumeration) must equal the oracle's
bit for bit; the work is integer-only, so there is no tolerance.
Sources: "Batched leaf-mask topology construction for generated conv grids"
(PR page) sections 1 and 2, Test plan (mixed member sizes, empty members first /
middle / last / all, coordinates straddling +-4096 tiles and negative octants,
factors 2 and 4, k3s2 transpose, refine->coarsen round trip).
"""
import itertools

import numpy as np
import pytest

import oracle
from tests.gpu_util import assert_same, gpu_build, gpu_fields, headers_as_oracle
from topology_construction_amd import synth

pytestmark = pytest.mark.gpu

OPS = [("coarsen", 2), ("refine", 2), ("dilate", 1), ("pad_neg", 1), ("pad_pos", 1), ("conv_t_k3s2", 2),
       ("coarsen", 4), ("coarsen", 8), ("refine", 4)]


def _check(op, f, ijk, off, ctx=""):
    print(f"[parity] {ctx} op={op} f={f} B={len(off) - 1} N={int(off[-1])}", flush=True)
    ref = oracle.run_threaded(op, f, ijk, off)
    batch, _ = gpu_build(op, f, ijk, off)
    assert_same(gpu_fields(batch), ref, f"{ctx} {op}x{f}")


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_from_ijk_matches_oracle(cfg):
    ijk, off = synth.make_config(cfg)
    _check("identity", 1, ijk, off, f"config{cfg}")


def test_from_ijk_unsorted_duplicated_rows():
    ijk, off = synth.make_config(1)
    rng = np.random.default_rng(5)
    members = []
    for g in range(len(off) - 1):
        m = ijk[off[g]:off[g + 1]]
        m = np.concatenate([m, m[: len(m) // 3]])  # duplicates collapse
        members.append(m[rng.permutation(len(m))])
    ijk2, off2 = synth.concat_members(members)
    _check("identity", 1, ijk2, off2, "shuffled+dup")


def test_from_ijk_scattered_rows():
    """Rows too far apart to share a packed key (more than 2^15 in x, leaf y or
    leaf z from their chunk's first row) take the front-end's unpacked path, one
    record per run; clustered members beside them take the packed one."""
    rng = np.random.default_rng(11)
    members = []
    for g in range(6):
        if g % 2 == 0:  # scattered over +-2^28, in arbitrary order, with repeats
            m = rng.integers(-(1 << 28), 1 << 28, size=(3000, 3))
            m = np.concatenate([m, m[:500]])
        else:  # a clustered blob in the same batch
            m = rng.integers(0, 40, size=(3000, 3)) + rng.integers(-(1 << 20), 1 << 20, size=3)
        members.append(m[rng.permutation(len(m))].astype(np.int32))
    ijk, off = synth.concat_members(members)
    _check("identity", 1, ijk, off, "scattered")
    _check("dilate", 1, ijk, off, "scattered")


def test_from_ijk_tile_table_rerun():
    """More distinct root tiles (36^3 = 46656) than the front-end's first tile
    table takes at half load (2^15): the record pass runs again with a table
    sized by its record count."""
    t = np.arange(36) * 4096 - 18 * 4096
    X, Y, Z = np.meshgrid(t, t, t, indexing="ij")
    v = np.stack([X.ravel(), Y.ravel(), Z.ravel()], axis=1) + np.array([5, 1, 3])
    rng = np.random.default_rng(12)
    v = v[rng.permutation(len(v))].astype(np.int32)
    ijk, off = synth.concat_members([v[:20000], v[20000:]])
    _check("identity", 1, ijk, off, "many tiles")


@pytest.mark.parametrize("op,f", OPS)
def test_config1_ops(op, f):
    ijk, off = synth.make_config(1)
    _check(op, f, ijk, off, "config1")


@pytest.mark.parametrize("op,f", [("coarsen", 2), ("refine", 2), ("dilate", 1), ("conv_t_k3s2", 2)])
def test_config2_ops(op, f):
    ijk, off = synth.make_config(2)
    _check(op, f, ijk, off, "config2")


@pytest.mark.parametrize("op,f", [("coarsen", 2), ("refine", 2), ("dilate", 1), ("pad_neg", 1), ("pad_pos", 1),
                                  ("refine", 4), ("conv_t_k3s2", 2), ("coarsen", 4)])
def test_config3_mixed_straddling_empty(op, f):
    ijk, off = synth.make_config(3)
    _check(op, f, ijk, off, "config3")


@pytest.mark.parametrize("op", ["conv_s1", "conv_t_s1"])
@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_kernel_k_stride1(op, k):
    # PR page section 2 / test plan: conv and transposed conv, K in {2,3,4,5} at
    # stride 1, as box-pass sequences (K = 1 copies the source)
    ijk, off = synth.make_config(3)
    _check(op, k, ijk, off, "config3")


@pytest.mark.parametrize("op", ["conv_s1", "conv_t_s1"])
def test_kernel_k_stride1_config2_k8_and_empty(op):
    ijk, off = synth.make_config(2)
    _check(op, 8, ijk, off, "config2")
    members = [np.zeros((0, 3), np.int32), np.array([[5, -4097, 4095]], np.int32), np.zeros((0, 3), np.int32)]
    ijk2, off2 = synth.concat_members(members)
    _check(op, 4, ijk2, off2, "single voxel between empties")


def _voxel_total(ijk, off):
    return int(oracle.run("identity", 1, ijk, off, fields=["headers"])["headers"][:, 8].sum())


@pytest.mark.parametrize("cfg,f", [(1, 2), (2, 2), (3, 2), (3, 4), (1, 8)])
def test_masked_refine(cfg, f):
    # PR page test plan: masked refine (per-voxel keep flags, then refine)
    import torch
    from topology_construction_amd import binding
    ijk, off = synth.make_config(cfg)
    keep = (np.random.default_rng(700 + cfg).random(_voxel_total(ijk, off)) < 0.6).astype(np.uint8)
    print(f"[parity] masked refine config{cfg} f={f} kept={int(keep.sum())}/{keep.size}", flush=True)
    ref = oracle.run_masked_refine(f, ijk, off, keep)
    _, src = gpu_build("identity", 1, ijk, off)
    out = binding.tc_build_masked_refine(src, torch.from_numpy(keep).cuda(), f)
    assert_same(gpu_fields(out), ref, f"masked refine config{cfg} x{f}")


def test_masked_refine_all_none_and_bad_length():
    import torch
    from topology_construction_amd import binding
    ijk, off = synth.make_config(3)
    n = _voxel_total(ijk, off)
    _, src = gpu_build("identity", 1, ijk, off)
    full = binding.tc_build_masked_refine(src, torch.ones(n, dtype=torch.uint8, device="cuda"), 2)
    assert_same(gpu_fields(full), oracle.run("refine", 2, ijk, off), "all kept")
    none = binding.tc_build_masked_refine(src, torch.zeros(n, dtype=torch.bool, device="cuda"), 2)
    assert_same(gpu_fields(none), oracle.run_masked_refine(2, ijk, off, np.zeros(n, np.uint8)), "none kept")
    for bad in (n - 1, n + 1):
        with pytest.raises(binding.TopoError) as e:
            binding.tc_build_masked_refine(src, torch.ones(bad, dtype=torch.uint8, device="cuda"), 2)
        assert e.value.status == binding.TC_ERR_INVALID_ARG


CENTRES = [(0, 0, 0), (4096, 0, -4096), (-4096, 4095, 127), (-1, -1, -1), (130, -130, 8), (-8192, 8191, 0)]


def _random_members(seed, n_members, max_vox):
    rng = np.random.default_rng(seed)
    members = []
    for _ in range(n_members):
        k = int(rng.integers(0, max_vox + 1))
        c = np.array(CENTRES)[rng.integers(0, len(CENTRES), size=k)]
        members.append((c + rng.integers(-20, 21, size=(k, 3))).astype(np.int32))
    return synth.concat_members(members)


@pytest.mark.parametrize("op,f", OPS + [("identity", 1)])
def test_random_sparse_members(op, f):
    ijk, off = _random_members(77, 6, 300)
    _check(op, f, ijk, off, "random")


def _many_members(seed, B, max_vox):
    """B small members (0..max_vox voxels each, about one in eight empty), each a
    cloud around its own centre spread over +-3000, so that members straddle root
    tiles and sign changes."""
    rng = np.random.default_rng(seed)
    members = []
    for _ in range(B):
        k = 0 if rng.random() < 0.125 else int(rng.integers(1, max_vox + 1))
        c = rng.integers(-3000, 3001, size=3)
        members.append((c + rng.integers(-12, 13, size=(k, 3))).astype(np.int32))
    return synth.concat_members(members)


@pytest.mark.parametrize("B", [300, 4200])
def test_many_members(B):
    """Batches past the per-batch LDS tables: grid voxel begins read from global
    memory in the enumeration (above 256 members), the multi-launch finalize path
    (above 1024) and the ijk front end's global member search (above 4095)."""
    ijk, off = _many_members(900 + B, B, 24)
    for op, f in [("identity", 1), ("coarsen", 2), ("refine", 2), ("dilate", 1), ("pad_pos", 1),
                  ("conv_t_k3s2", 2)]:
        _check(op, f, ijk, off, f"many members B={B}")


def test_octant_corners_of_root_tile():
    corners = np.array([(a, b, c) for a in (0, 4095) for b in (0, 4095) for c in (0, 4095)], np.int32)
    across = corners + np.where(corners > 0, 1, -1).astype(np.int32) * np.array([1, 0, 0], np.int32)
    ijk, off = synth.concat_members([corners, across, corners - 4096])
    for op, f in OPS:
        _check(op, f, ijk, off, "corners")


def _face_members():
    """One member per placement of a voxel on (or one voxel inside) a face, edge or
    corner of its lower node (128 voxels) and of its root tile (4096 voxels), on
    both sides of 0 and of +-4096, each with a voxel in the node's middle too."""
    members = []
    bases = [(0, 0, 0), (128 * 5, 0, 256), (4096, -4096, 0), (-128, -4096 * 2, 4096 * 3)]
    for bx, by, bz in bases:
        for side in (0, 127, 1, 126):
            for axes in ((0,), (1,), (2,), (0, 1), (1, 2), (0, 2), (0, 1, 2)):
                v = [64, 64, 64]
                for a in axes:
                    v[a] = side
                members.append(np.array([[bx + v[0], by + v[1], bz + v[2]], [bx + 64, by + 64, bz + 64]], np.int32))
    for t in (0, 4095, 1, 4094):  # root-tile faces: the lower at the tile's end
        for axes in ((0,), (1,), (2,), (0, 1, 2)):
            v = [2048, 2048, 2048]
            for a in axes:
                v[a] = t
            members.append(np.array([v, [2048, 2048, 2048]], np.int32))
            members.append(np.array(v, np.int32)[None, :] - 4096)
    # batches of 24 members keep every batch on the one-workgroup path (at most
    # 75 source lowers for a box op), where the face test is made
    return [synth.concat_members(members[i:i + 24]) for i in range(0, len(members), 24)]


@pytest.mark.parametrize("op,f", [("dilate", 1), ("pad_neg", 1), ("pad_pos", 1), ("conv_t_k3s2", 2)])
def test_box_ops_voxels_on_node_faces(op, f):
    """Box ops prune neighbour tiles and lowers by which faces hold a voxel: a
    voxel on a face, edge or corner must still reach every neighbour, one voxel
    inside must reach none (PR page, section 2: box-dilate and pads)."""
    for n, (ijk, off) in enumerate(_face_members()):
        _check(op, f, ijk, off, f"faces batch {n}")


def _solid_members():
    """Dense sources: solid cubes of 8^3 full leaves against the low and the high
    faces of a lower (its interior leaves and its face leaves next to outside
    positions), a solid cube across lower and root-tile boundaries at negative
    coordinates, a two-voxel slab, and an empty member."""
    g = np.mgrid[0:120, 0:120, 0:2].reshape(3, -1).T
    slab = (g + np.array([-100, 37, 5])).astype(np.int32)
    return synth.concat_members([synth.cube_voxels(64, (0, 0, 0)), synth.cube_voxels(64, (64, 64, 64)),
                                 np.zeros((0, 3), np.int32), synth.cube_voxels(40, (-4115, -20, 4080)), slab])


@pytest.mark.parametrize("op,f", [("dilate", 1), ("pad_neg", 1), ("pad_pos", 1)])
def test_box_ops_solid_sources(op, f):
    """Box ops on dense sources: a lower whose leaves are all present (its
    interior leaves spill only onto marked positions), dense runs of candidates
    and faces of full neighbours (PR page, section 2: box-dilate and pads)."""
    ijk, off = _solid_members()
    _check(op, f, ijk, off, "solid")


@pytest.mark.parametrize("op,f", [("dilate", 1), ("pad_neg", 1), ("pad_pos", 1), ("conv_t_k3s2", 2)])
def test_box_ops_wide_address_form(op, f):
    """The box ops' leaf gather in the form batches with source arrays of 2 GiB or
    more take (64-bit addresses), forced on small inputs: same results."""
    from topology_construction_amd import binding
    binding.tc_debug_wide_loads(True)
    try:
        ijk, off = synth.make_config(3)
        _check(op, f, ijk, off, "wide config 3")
        ijk, off = _solid_members()
        _check(op, f, ijk, off, "wide solid")
    finally:
        binding.tc_debug_wide_loads(False)


@pytest.mark.parametrize("op", ["conv_s1", "conv_t_s1"])
@pytest.mark.parametrize("k", [2, 4, 5])
def test_kernel_k_voxels_on_node_faces(op, k):
    for n, (ijk, off) in enumerate(_face_members()):
        _check(op, k, ijk, off, f"faces batch {n}")


def test_empty_members_everywhere():
    ijk, off = synth.make_config(1)
    a, b = ijk[off[0]:off[1]], ijk[off[1]:off[2]]
    e = np.zeros((0, 3), np.int32)
    ijk2, off2 = synth.concat_members([e, a, e, e, b, e])
    for op, f in OPS:
        _check(op, f, ijk2, off2, "empties")


def test_all_members_empty_and_single_empty():
    import torch
    from topology_construction_amd import binding
    for B in (1, 4):
        off = np.zeros(B + 1, np.int64)
        ijk = np.zeros((0, 3), np.int32)
        for op, f in OPS + [("identity", 1)]:
            _check(op, f, ijk, off, f"all-empty B={B}")


def test_int32_limits():
    from topology_construction_amd import binding
    ok = (1 << 30) - 1
    ijk = np.array([[ok, -ok - 1, 0], [ok, ok, ok]], np.int32)
    _check("refine", 2, ijk, np.array([0, 2]), "refine at 2^30-1")
    for bad in ([[1 << 30, 0, 0]], [[0, -(1 << 30) - 1, 0]]):
        batch_src, _ = gpu_build("identity", 1, np.array(bad, np.int32), np.array([0, 1]))
        with pytest.raises(binding.TopoError) as e:
            binding.tc_build_batched_topology(batch_src, "refine", 2)
        assert e.value.status == binding.TC_ERR_OVERFLOW
    top = np.array([[0, 0, (1 << 31) - 1], [-(1 << 31), 5, 5]], np.int32)
    src, _ = gpu_build("identity", 1, top, np.array([0, 2]))
    for op in ("dilate", "pad_pos", "pad_neg"):
        with pytest.raises(binding.TopoError) as e:
            binding.tc_build_batched_topology(src, op, 1)
        assert e.value.status == binding.TC_ERR_OVERFLOW
    _check("pad_neg", 1, top[:1], np.array([0, 1]), "pad_neg at INT32_MAX")
    _check("pad_pos", 1, top[1:], np.array([0, 1]), "pad_pos at INT32_MIN")
    _check("coarsen", 8, top, np.array([0, 2]), "coarsen at limits")


def test_many_tiles_large_sort_paths():
    # > 4096 unique tiles (from_ijk) and > 4096 tile candidates (dilate: 27 per upper)
    rng = np.random.default_rng(9)
    pts = rng.integers(-(1 << 28), 1 << 28, size=(6000, 3)).astype(np.int32)
    ijk, off = synth.concat_members([pts[:2500], pts[2500:2600], pts[2600:]])
    for op, f in [("identity", 1), ("dilate", 1), ("refine", 2), ("coarsen", 2)]:
        _check(op, f, ijk, off, "many-tiles")


def _tiles_members(seed, B, tiles_per_member, span):
    """B members, each with one voxel in every one of `tiles_per_member` distinct
    root tiles drawn from [-span, span]^3 (tile units)."""
    rng = np.random.default_rng(seed)
    members = []
    for _ in range(B):
        t = np.unique(rng.integers(-span, span + 1, size=(tiles_per_member * 2, 3)), axis=0)[:tiles_per_member]
        members.append((t * 4096 + rng.integers(0, 4096, size=t.shape)).astype(np.int32))
    return synth.concat_members(members)


@pytest.mark.parametrize("seed,B,per,span", [
    (21, 8, 20, 2),     # compact tile ranges: the LDS bitmap over (grid, tile) keys
    (22, 6, 25, 400),   # 64 < keys, at most 128 per grid, key space too large for the bitmap: per-grid rank
    (23, 8, 60, 400),   # several hundred keys, at most 128 per grid: the per-grid rank sort
    (24, 8, 150, 400),  # more than 1024 keys: the LDS bitonic network
    (25, 1, 200, 400),  # one grid above 128 keys (no per-grid rank), at most 256 keys: the rank sort
    (26, 2, 300, 400),  # grids above 128 keys, 256 < keys <= 1024: the one-key-per-thread bitonic network
])
def test_tile_dedup_paths(seed, B, per, span):
    """Every tile-dedup path of the one-workgroup tile stage (4096 candidates at
    most) against the oracle."""
    ijk, off = _tiles_members(seed, B, per, span)
    for op, f in [("coarsen", 2), ("refine", 2), ("dilate", 1)]:
        _check(op, f, ijk, off, f"tiles seed={seed}")


def test_pyramid_chain_config4():
    """Coarsen x2 three times, then k3s2 transpose back up, each level from the GPU output."""
    from topology_construction_amd import binding
    ijk, off = synth.make_config(4)
    batch, src = gpu_build("identity", 1, ijk, off)
    levels = [batch]
    ref_ijk, ref_off = ijk, off
    for lvl in range(3):
        ref = oracle.run_threaded("coarsen", 2, ref_ijk, ref_off)
        nxt = binding.tc_build_batched_topology(levels[-1], "coarsen", 2)
        assert_same(gpu_fields(nxt), ref, f"pyramid coarsen level {lvl + 1}")
        levels.append(nxt)
        ref_ijk, ref_off = ref["ijk"], np.concatenate([[0], np.cumsum(ref["headers"][:, 8])])
    cur = levels[-1]
    for lvl in range(3):
        ref = oracle.run_threaded("conv_t_k3s2", 2, ref_ijk, ref_off)
        cur = binding.tc_build_batched_topology(cur, "conv_t_k3s2", 2)
        assert_same(gpu_fields(cur), ref, f"pyramid k3s2T level {lvl + 1}")
        ref_ijk, ref_off = ref["ijk"], np.concatenate([[0], np.cumsum(ref["headers"][:, 8])])
    # single calls at factors 4 and 8 on every member (refine x8: ~58M voxels)
    for op, f in [("refine", 4), ("refine", 8), ("coarsen", 4), ("coarsen", 8)]:
        _check(op, f, ijk, off, "config4")


def test_null_allocator_path():
    """Outputs from hipMallocAsync (no torch allocator): headers and ijk still match."""
    import torch
    from tests.gpu_util import headers_as_oracle
    from topology_construction_amd import binding
    ijk, off = synth.make_config(3)
    t = torch.from_numpy(ijk).cuda()
    src = binding.tc_batch_from_ijk(t, off, allocator="none")
    for op, f in [("dilate", 1), ("refine", 2)]:
        out = binding.tc_build_batched_topology(src, op, f, allocator="none")
        ref = oracle.run(op, f, ijk, off, fields=["headers", "ijk"])
        assert np.array_equal(headers_as_oracle(out.headers()), ref["headers"])
        assert np.array_equal(out.ijk().cpu().numpy(), ref["ijk"])


def test_deterministic_bits():
    ijk, off = synth.make_config(3)
    for op, f in [("dilate", 1), ("coarsen", 2)]:
        a, src = gpu_build(op, f, ijk, off)
        from topology_construction_amd import binding
        b = binding.tc_build_batched_topology(src, op, f)
        fa, fb = gpu_fields(a), gpu_fields(b)
        for k in fa:
            assert np.array_equal(fa[k], fb[k]), k


def test_scratch_cache_reuse_and_release():
    """Passes reuse the process-wide cached scratch blocks; results stay the
    same when blocks are reused by a different op (stale contents), after they
    are released, and on another stream."""
    import torch
    from topology_construction_amd import binding
    ijk, off = synth.make_config(3)
    ref = {op: oracle.run(op, f, ijk, off) for op, f in [("dilate", 1), ("refine", 2)]}
    src = binding.tc_batch_from_ijk(torch.from_numpy(ijk).cuda(), off)
    for op, f in [("dilate", 1), ("refine", 2), ("dilate", 1)]:
        assert_same(gpu_fields(binding.tc_build_batched_topology(src, op, f)), ref[op], f"reuse {op}")
    binding.tc_scratch_release()
    assert_same(gpu_fields(binding.tc_build_batched_topology(src, "refine", 2)), ref["refine"], "after release")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = binding.tc_build_batched_topology(src, "dilate", 1, stream=s)
    s.synchronize()
    assert_same(gpu_fields(out), ref["dilate"], "second stream")
    # batch buffers of the library's own allocation go back to its cache on free
    # and are taken again by the next batch that fits (stale contents)
    # (field views need torch-owned buffers: compare headers and the enumeration)
    def same_ijk_headers(b, r, what):
        assert np.array_equal(headers_as_oracle(b.headers()), r["headers"]), what
        assert np.array_equal(b.ijk().cpu().numpy(), r["ijk"]), what

    for op, f in [("refine", 2), ("dilate", 1), ("refine", 2)]:
        b = binding.tc_build_batched_topology(src, op, f, allocator="none")
        same_ijk_headers(b, ref[op], f"cached buffer {op}")
        del b
    binding.tc_scratch_release()
    same_ijk_headers(binding.tc_build_batched_topology(src, "dilate", 1, allocator="none"), ref["dilate"],
                     "after release")
    torch.cuda.synchronize()


def test_self_consistency_from_ijk_of_enumeration():
    """from_ijk(enumerate(op(g))) == op(g) elementwise (the pages' pinning method)."""
    from topology_construction_amd import binding
    ijk, off = synth.make_config(3)
    for op, f in [("dilate", 1), ("refine", 2), ("coarsen", 2)]:
        out, _ = gpu_build(op, f, ijk, off)
        fo = gpu_fields(out)
        h = fo["headers"]
        re, _ = gpu_build("identity", 1, fo["ijk"], np.concatenate([[0], np.cumsum(h[:, 8])]))
        fr = gpu_fields(re)
        for k in fo:
            assert np.array_equal(fo[k], fr[k]), (op, k)
