"""Host-side checks of bench.py that need no GPU: the one-GPU refusal, the
algorithmic byte formulas behind the roofline, and the source digest that decides
whether committed counter traffic still describes the kernels."""
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    line = [ln for ln in r.stdout.splitlines() if ln.startswith("{")][-1]
    assert "one GPU" in json.loads(line)["error"]


def test_kernel_bytes():
    # enumeration: origin, mask, offset and grid base per leaf (96 B), 12 B per voxel
    assert bench.kernel_bytes("k_enumerate", 7, 3, 100) == 96 * 3 + 12 * 100
    # marking reads each source leaf's origin and mask once
    assert bench.kernel_bytes("k_leaf_mark_lower", 5, 40, 999) == 80 * 5
    assert bench.kernel_bytes("k_leaf_mark_box", 5, 40, 999) == 80 * 5
    # gather: per output leaf origin + candidate id + written mask, per source leaf its mask
    assert bench.kernel_bytes("k_leaf_gather", 5, 40, 999) == 84 * 40 + 64 * 5
    assert bench.kernel_bytes("k_finalize_small", 5, 40, 999) == 36 * 40
    with pytest.raises(ValueError):
        bench.kernel_bytes("k_unknown", 1, 1, 1)


@pytest.fixture()
def tree_copy(tmp_path, monkeypatch):
    """A copy of the kernel sources and committed profiles, with bench reading it."""
    for sub in (os.path.join("topology_construction_amd", "csrc"), "profiles"):
        shutil.copytree(os.path.join(ROOT, sub), tmp_path / sub)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path


def _edit(path, old, new):
    text = path.read_text()
    assert old in text
    path.write_text(text.replace(old, new, 1))


def test_digest_ignores_comments_but_not_code(tree_copy):
    base = bench.source_digest()
    src = tree_copy / "topology_construction_amd" / "csrc" / "tree.hip"
    _edit(src, "constexpr int kEnumMaxLeaves = 8;", "constexpr int kEnumMaxLeaves = 8;  // a comment\n\n")
    assert bench.source_digest() == base
    _edit(src, "constexpr int kEnumMaxLeaves = 8;", "constexpr int kEnumMaxLeaves = 4;")
    assert bench.source_digest() != base


def test_recorded_traffic_follows_the_digest(tree_copy):
    rec = tree_copy / "profiles" / "traffic_k_enumerate_shells_b16_res64.txt"
    kv = dict(ln.split(None, 1) for ln in rec.read_text().splitlines() if ln and not ln.startswith("#"))
    if kv.get("source_sha256") != bench.source_digest():
        pytest.skip("the committed traffic summary predates the current kernel sources")
    assert bench.recorded_traffic("k_enumerate", "shells_b16_res64") == float(kv["hbm_bytes_per_launch"])
    _edit(tree_copy / "topology_construction_amd" / "csrc" / "tree.hip", "constexpr int kEnumMaxLeaves = 8;",
          "constexpr int kEnumMaxLeaves = 4;")
    assert bench.recorded_traffic("k_enumerate", "shells_b16_res64") is None
    assert bench.recorded_traffic("k_enumerate", "no_such_workload") is None
