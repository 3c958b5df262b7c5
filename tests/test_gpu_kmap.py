"""Kernel maps on the GPU vs the oracle, element by element, through the C ABI.

Issue page "Generated-topology grid construction dominates per-iteration
ConvolutionPlan cost (serial per-grid build + merge)", Measurements: a plan
builds a k3 s1 kernel map on one topology and a k2s2 transposed-conv map. Both,
and the other kernel sizes and strides the library accepts, must equal the
oracle's table bit for bit (integer work, no tolerance), including members that
are empty, straddle the +-4096 root tiles or sit in negative octants, rows with
no source at all, and coordinates at the ends of int32.
"""
import numpy as np
import pytest

import oracle
from tests.gpu_util import gpu_build
from topology_construction_amd import synth

pytestmark = pytest.mark.gpu


def _oracle_batches(src_op, dst_op, ijk, off):
    src = oracle.run(src_op[0], src_op[1], ijk, off, fields=["headers", "ijk"])
    dst = oracle.run(dst_op[0], dst_op[1], ijk, off, fields=["headers", "ijk"])
    return src, dst


def _check(ijk, off, dst_op, k, s, transposed, ctx, src_op=("identity", 1)):
    from topology_construction_amd import binding
    print(f"[kmap] {ctx} dst={dst_op} K={k} S={s} T={int(transposed)} B={len(off) - 1} N={int(off[-1])}",
          flush=True)
    src_ref, dst_ref = _oracle_batches(src_op, dst_op, ijk, off)
    ref = oracle.kernel_map(src_ref, dst_ref, k, s, transposed)
    src, _ = gpu_build(src_op[0], src_op[1], ijk, off)
    dst, _ = gpu_build(dst_op[0], dst_op[1], ijk, off, src=None if src_op != ("identity", 1) else src)
    got = binding.tc_build_kernel_map(src, dst, k, s, transposed).cpu().numpy()
    assert got.shape == ref.shape, (ctx, got.shape, ref.shape)
    if not np.array_equal(got, ref):
        bad = np.argwhere(got != ref)
        raise AssertionError(f"{ctx}: {bad.shape[0]} mismatches, first at {bad[:3].tolist()}: "
                             f"gpu {got[tuple(bad[0])]} oracle {ref[tuple(bad[0])]}")
    return got


# the two maps the issue page measures, on the configurations it measures them at
@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_same_topology_k3s1(cfg):
    ijk, off = synth.make_config(cfg)
    _check(ijk, off, ("identity", 1), 3, 1, False, f"config{cfg}")


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_transposed_k2s2_onto_refine(cfg):
    ijk, off = synth.make_config(cfg)
    _check(ijk, off, ("refine", 2), 2, 2, True, f"config{cfg}")


@pytest.mark.parametrize("cfg", [1, 3])
def test_conv_k2s2_onto_coarsen_and_k3s2_transposed(cfg):
    ijk, off = synth.make_config(cfg)
    _check(ijk, off, ("coarsen", 2), 2, 2, False, f"config{cfg}")
    _check(ijk, off, ("conv_t_k3s2", 2), 3, 2, True, f"config{cfg}")


def _workload(name):
    """config 1, config 3, or a slice of config 3 (members 0-5, with the empty
    member 0 and members translated across root tiles, plus the empty member 24)
    that keeps K^3-wide oracle tables small."""
    if name == "config1":
        return synth.make_config(1)
    ijk, off = synth.make_config(3)
    if name == "config3":
        return ijk, off
    keep = list(range(6)) + [24]
    return synth.concat_members([ijk[off[g]:off[g + 1]] for g in keep])


@pytest.mark.parametrize("k,transposed,where", [(1, False, "config3"), (2, False, "config3"), (2, True, "config3"),
                                                (4, False, "config3 slice"), (4, True, "config3 slice"),
                                                (5, False, "config3 slice"), (5, True, "config3 slice"),
                                                (8, False, "config1"), (8, True, "config1")])
def test_stride1_kernel_k(k, transposed, where):
    ijk, off = _workload(where)
    _check(ijk, off, ("conv_t_s1" if transposed else "conv_s1", k), k, 1, transposed, where)


@pytest.mark.parametrize("k,transposed,where", [(3, False, "config3"), (8, False, "config3 slice"),
                                                (4, True, "config3 slice"), (8, True, "config1")])
def test_stride2_wide_regions(k, transposed, where):
    # the k8 s2 conv reads a 22^3 region per target leaf (the single-wave launch)
    ijk, off = _workload(where)
    _check(ijk, off, ("coarsen", 2) if not transposed else ("refine", 2), k, 2, transposed, where)


def test_unrelated_target_rows_without_sources():
    # target = the dilation of the source: many rows read nothing for a k2 kernel
    ijk, off = synth.make_config(1)
    _check(ijk, off, ("dilate", 1), 2, 1, False, "config1")
    _check(ijk, off, ("dilate", 1), 2, 2, True, "config1")
    _check(ijk, off, ("coarsen", 4), 3, 2, False, "config1")


def _members(sets):
    return synth.concat_members([np.array(sorted(s), np.int32).reshape(-1, 3) for s in sets])


def test_empty_members_and_straddling_tiles():
    rng = np.random.default_rng(77)
    sets = [set(), {(4095, -1, 0), (4096, 0, -4097), (-4096, 4095, 7)}, set(),
            {(int(a), int(b), int(c)) for a, b, c in rng.integers(-40, 40, size=(300, 3))}, set()]
    ijk, off = _members(sets)
    for k, s, t, op in [(3, 1, False, ("identity", 1)), (2, 2, True, ("refine", 2)), (2, 2, False, ("coarsen", 2)),
                        (5, 1, True, ("conv_t_s1", 5))]:
        _check(ijk, off, op, k, s, t, "empty+straddle")


def test_int32_ends():
    hi, lo = (1 << 31) - 1, -(1 << 31)
    sets = [{(hi, hi, hi), (hi - 1, hi, hi - 8), (hi - 9, hi - 3, hi)},
            {(lo, lo, lo), (lo + 1, lo, lo + 8), (lo + 9, lo + 3, lo)}]
    ijk, off = _members(sets)
    _check(ijk, off, ("identity", 1), 3, 1, False, "int32 ends")
    _check(ijk, off, ("identity", 1), 8, 1, True, "int32 ends")
    _check(ijk, off, ("coarsen", 2), 3, 2, False, "int32 ends")
    _check(ijk, off, ("identity", 1), 4, 2, True, "int32 ends")


def test_all_members_empty_and_argument_errors():
    import torch
    from topology_construction_amd import binding
    ijk, off = _members([set(), set()])
    e, _ = gpu_build("identity", 1, ijk, off)
    m = binding.tc_build_kernel_map(e, e, 3, 1, False)
    assert tuple(m.shape) == (0, 27)
    ijk1, off1 = synth.make_config(1)
    a, _ = gpu_build("identity", 1, ijk1, off1)
    one, _ = gpu_build("identity", 1, ijk1[:5], np.array([0, 5], np.int64))
    with pytest.raises(binding.TopoError) as ex:
        binding.tc_build_kernel_map(a, one, 3, 1, False)
    assert ex.value.status == 1
    for k, s, st in [(0, 1, 1), (9, 1, 1), (3, 0, 1), (3, 3, 5)]:
        with pytest.raises(binding.TopoError) as ex:
            binding.tc_build_kernel_map(a, a, k, s, False)
        assert ex.value.status == st, (k, s)
    small = torch.empty(10, dtype=torch.int32, device="cuda")
    with pytest.raises(binding.TopoError) as ex:
        binding.tc_build_kernel_map(a, a, 3, 1, False, out=small)
    assert ex.value.status == 1
    torch.cuda.synchronize()
