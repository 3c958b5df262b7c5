"""Planted mistakes in the oracle must be caught by its pins.

Each case copies oracle/oracle.cpp, changes one line the way a plausible slip
would (a transposed operand, a dropped or wrong term, a wrong sign or index, an
off-by-one), compiles the copy with g++ on the CPU and runs the pin battery of
test_oracle_pins.py against it. The battery must fail for every mutant; the
unmodified oracle passes it (that is test_oracle_pins.py itself).
"""
import functools
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

MUTANTS = {
    "leaf bit x/y swapped": ("const i64 n = k[9] * 64 + k[10] * 8 + k[11];",
                             "const i64 n = k[10] * 64 + k[9] * 8 + k[11];"),
    "coarsen truncates": ("out.push_back({floordiv(v.x, factor), floordiv(v.y, factor), floordiv(v.z, factor)});",
                          "out.push_back({v.x / factor, floordiv(v.y, factor), floordiv(v.z, factor)});"),
    "refine sign": ("out.push_back({v.x * factor + dx, v.y * factor + dy, v.z * factor + dz});",
                    "out.push_back({v.x * factor - dx, v.y * factor + dy, v.z * factor + dz});"),
    "pad_neg box": ("case OP_PAD_NEG: box(-1, 0, in); break;", "case OP_PAD_NEG: box(0, 1, in); break;"),
    "dilate box": ("case OP_DILATE: box(-1, 1, in); break;", "case OP_DILATE: box(-1, 0, in); break;"),
    "k3s2 pad side": ("box(-1, 0, fine);", "box(0, 1, fine);"),
    "tile axes transposed": ("k[a] = floordiv(c[a], 4096);", "k[2 - a] = floordiv(c[a], 4096);"),
    "leaf prefix off by one": ("run += (u64)popcount64(r->leaf_mask[l * 8 + w - 1]);",
                               "run += (u64)popcount64(r->leaf_mask[l * 8 + w]);"),
    "lower prefix inclusive": ("r->lower_prefix[l * 64 + w] = (uint16_t)run;\n        run += popcount64(r->lower_mask[l * 64 + w]);",
                               "run += popcount64(r->lower_mask[l * 64 + w]);\n        r->lower_prefix[l * 64 + w] = (uint16_t)run;"),
    "bbox operand": ("bmin[a] = std::min(bmin[a], c[a]);", "bmin[a] = std::min(bmin[a], c[(a + 1) % 3]);"),
    "root key axes": ("r->upper_key.push_back((ux << 40) | (uy << 20) | uz);",
                      "r->upper_key.push_back((uz << 40) | (uy << 20) | ux);"),
    "upper child bit": ("const i64 bit = (k[3] * 32 + k[4]) * 32 + k[5];",
                        "const i64 bit = (k[5] * 32 + k[4]) * 32 + k[3];"),
    "lower child bit": ("const i64 bit = (k[6] * 16 + k[7]) * 16 + k[8];",
                        "const i64 bit = (k[6] * 16 + k[8]) * 16 + k[7];"),
    "voxel begin": ("h[9] = voxel_total;", "h[9] = 0;"),
    "leaf offset base": ("r->leaf_offset.push_back(nvox);", "r->leaf_offset.push_back(nvox + 1);"),
    "upper first child": ("r->upper_first.push_back((int32_t)r->lower_first.size());",
                          "r->upper_first.push_back((int32_t)r->leaf_parent.size());"),
    "lower parent": ("(int32_t)(k[2] * 4096 + k[5] * 128), (int32_t)upper_idx});",
                     "(int32_t)(k[2] * 4096 + k[5] * 128), (int32_t)g});"),
    "overflow z unchecked": ("if (!in_int32(v.x) || !in_int32(v.y) || !in_int32(v.z)) return false;",
                             "if (!in_int32(v.x) || !in_int32(v.y)) return false;"),
    "conv_s1 leans the wrong way": ("case OP_CONV_S1: box(-(factor / 2), (factor - 1) / 2, in); break;",
                                    "case OP_CONV_S1: box(-((factor - 1) / 2), factor / 2, in); break;"),
    "masked refine inverts the mask": ("        if (keep[j])\n", "        if (!keep[j])\n"),
    "kernel map transposed sign": ("const i64 q = o[a] - d[a];", "const i64 q = o[a] + d[a];"),
    "kernel map offsets z-major": ("const i64 d[3] = {lo + k / (K * K), lo + (k / K) % K, lo + k % K};",
                                   "const i64 d[3] = {lo + k % K, lo + (k / K) % K, lo + k / (K * K)};"),
    "kernel map box leans": ("const i64 lo = -((K - 1) / 2);\n  const i64 kk", "const i64 lo = -(K / 2);\n  const i64 kk"),
    "kernel map stride dropped": ("c[a] = (i64)S * o[a] + d[a];", "c[a] = o[a] + d[a];"),
    "kernel map inexact division kept": ("              if (floormod(q, S) != 0) exact = false;\n", ""),
    "kernel map members mix": ("for (i64 i = src_off[g]; i < src_off[g + 1]; ++i)\n        index[",
                               "for (i64 i = 0; i < src_off[B]; ++i)\n        index["),
    "conv_t_s1 box one short": ("case OP_CONV_T_S1: box(-((factor - 1) / 2), factor / 2, in); break;",
                                "case OP_CONV_T_S1: box(-((factor - 1) / 2), (factor - 1) / 2, in); break;"),
}

BATTERY = [
    functools.partial(pins.test_bruteforce_sets_and_order, "identity", 1),
    functools.partial(pins.test_bruteforce_sets_and_order, "coarsen", 2),
    functools.partial(pins.test_bruteforce_sets_and_order, "refine", 2),
    functools.partial(pins.test_bruteforce_sets_and_order, "dilate", 1),
    functools.partial(pins.test_bruteforce_sets_and_order, "pad_neg", 1),
    functools.partial(pins.test_bruteforce_sets_and_order, "conv_t_k3s2", 2),
    functools.partial(pins.test_bruteforce_sets_and_order, "conv_s1", 4),
    functools.partial(pins.test_bruteforce_sets_and_order, "conv_t_s1", 4),
    functools.partial(pins.test_masked_refine_bruteforce, 2),
    functools.partial(pins.test_refine_count_and_roundtrip, 2),
    pins.test_golden_canonical_order,
    pins.test_golden_tree_worked_example,
    functools.partial(pins.test_invariants_config1, "identity", 1),
    functools.partial(pins.test_invariants_config1, "dilate", 1),
    pins.test_invariants_random_sets,
    pins.test_overflow_and_limits,
    pins.test_golden_kernel_map,
    functools.partial(pins.test_kernel_map_bruteforce, 2, 1, True),
    functools.partial(pins.test_kernel_map_bruteforce, 3, 2, False),
    functools.partial(pins.test_kernel_map_bruteforce, 3, 2, True),
]


@pytest.fixture(scope="module")
def source():
    with open(oracle.SRC) as fh:
        return fh.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, source, tmp_path, monkeypatch):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation anchor not unique for {name!r}"
    src = tmp_path / "mutant.cpp"
    src.write_text(source.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["g++", "-O1", "-std=c++17", "-shared", "-fPIC", "-o", str(so), str(src)])
    lib = oracle.bind(str(so))
    monkeypatch.setattr(oracle, "run", functools.partial(oracle.run, lib=lib))
    monkeypatch.setattr(oracle, "run_masked_refine", functools.partial(oracle.run_masked_refine, lib=lib))
    monkeypatch.setattr(oracle, "kernel_map_rows", functools.partial(oracle.kernel_map_rows, lib=lib))
    failures = []
    for check in BATTERY:
        try:
            check()
        except (AssertionError, oracle.OracleError, KeyError, IndexError, ValueError,
                pytest.fail.Exception) as exc:
            failures.append((getattr(check, "__name__", str(check)), type(exc).__name__))
            break
    assert failures, f"mutant {name!r} passed every pin"


# Planted mistakes in the oracle's points front-end (Python): each must fail the
# points pins.
POINT_MUTANTS = {
    "points sign": ("x = (pts - org[g]) / vs[g]", "x = (org[g] - pts) / vs[g]"),
    "points scale": ("x = (pts - org[g]) / vs[g]", "x = (pts - org[g]) * vs[g]"),
    "points ties down": ("np.floor(x + np.float32(0.5)) if mode == 0", "np.ceil(x - np.float32(0.5)) if mode == 0"),
    "points mode 1 corners": ("for a in (0, 1) for b in (0, 1) for c in (0, 1)]",
                              "for a in (-1, 0) for b in (0, 1) for c in (0, 1)]"),
    "points member of row": ("g = np.repeat(np.arange(B), np.diff(off))", "g = np.zeros(off[-1], dtype=np.int64)"),
    "points origin axes": ("org = np.asarray(origin, dtype=np.float32).reshape(-1, 3)",
                           "org = np.asarray(origin, dtype=np.float32).reshape(-1, 3)[:, ::-1]"),
}


@pytest.mark.parametrize("name", sorted(POINT_MUTANTS))
def test_planted_points_mistake_is_caught(name, monkeypatch):
    import inspect
    old, new = POINT_MUTANTS[name]
    src = inspect.getsource(oracle.points_to_ijk)
    assert src.count(old) == 1, name
    ns = dict(oracle.__dict__)
    exec(src.replace(old, new), ns)
    monkeypatch.setattr(oracle, "points_to_ijk", ns["points_to_ijk"])
    battery = [pins.test_golden_points, functools.partial(pins.test_points_recover_jittered_centres, 0),
               functools.partial(pins.test_points_recover_jittered_centres, 1)]
    for check in battery:
        try:
            check()
        except (AssertionError, oracle.OracleError, ValueError, IndexError):
            return
    pytest.fail(f"points mutant {name!r} passed every pin")
