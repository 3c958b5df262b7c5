"""Benchmark of the batched topology hot path on one MI355X.

A step is one pass of the whole hot path over the B=16 resolution-64 shell
batch (16 ellipsoid shells, ~7.4k voxels each; it stands in for the pages'
shape-VAE workload of 16 shoes at resolution 64): conv k2s2 (coarsen x2),
k2s2 transpose (refine x2), k3s1 (box-dilate [-1,1]^3) and the chained k3s2
transpose (refine x2 then pad {-1,0}^3), built by one multi-target call, then
each target's jagged voxel enumeration. Inputs are resident in HBM before
timing starts.

Prints one JSON line (rank 0). `value` = output voxels per second over the K
timed steps. `roofline` reports the dominant kernel's algorithmic bytes per
launch over its HIP-event-timed average duration in those steps (and, beside
it, the same over its kernel-trace duration from the committed profile);
`ms_per_step_unprofiled` repeats the K steps without those events,
`ms_per_step_one_call_per_op` with one build call per op, and
`ms_per_step_torch_allocator` with torch's caching allocator supplying the
outputs (the step itself takes them from the library's pool, the C ABI's
default).
`cpu_baseline` times the CPU oracle on whole steps of the same workload, its
members spread over the host's threads (single-thread and 46M-voxel figures
beside it). Outside the timed steps the line also carries per-op medians
(`ops`, B=48 in `b48`, B=2 in `b2`), the pyramid chain and single-call factors
4 and 8 (`pyramid`), the stride-1 kernel-K targets and masked refine
(`more_ops`), the ijk and points front-ends (`from_ijk`, `from_points`), the
plan's kernel maps (`kernel_maps`) and the 46M-voxel batch (`large`).
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "output voxels/s & ms per batched pass (k2s2 refine/coarsen, k3s1 dilate), B=16/48"
STEP_OPS = [("coarsen", 2), ("refine", 2), ("dilate", 1), ("conv_t_k3s2", 2)]
HBM_PEAK_GBS = 8000.0
WORKLOAD_TAGS = {2: "shells_b16_res64", 5: "shells512_cubes"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, help="workload id (2: B=16 shells at res 64)")
    ap.add_argument("--roofline-kernel", default="k_enumerate")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-large", action="store_true", help="skip the 64-shell res-512 + cube batch")
    ap.add_argument("--large-only", action="store_true",
                    help="only the 64-shell res-512 + cube batch (prints its record), for profiling")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the run, copy a buffer of this many MiB device-to-device three times: "
                         "a kernel of known traffic that scales the HBM byte counters of a profiling run")
    return ap.parse_args()


def op_medians(binding, torch, np, src, reps=20):
    """Per-op pass and enumeration medians over `reps` runs (the Measurements
    protocol of the PR page: median of 20 timed iterations)."""
    ops = {}
    for op, f in STEP_OPS:
        pass_ms, enum_ms = [], []
        for _ in range(reps):
            torch.cuda.synchronize()
            a = time.perf_counter()
            out = binding.tc_build_batched_topology(src, op, f)
            torch.cuda.synchronize()
            b = time.perf_counter()
            ijk_out = binding.tc_enumerate_ijk(out)
            torch.cuda.synchronize()
            c = time.perf_counter()
            pass_ms.append((b - a) * 1e3)
            enum_ms.append((c - b) * 1e3)
        ops[f"{op}x{f}"] = {"ms_pass_median": float(np.median(pass_ms)),
                            "ms_enumerate_median": float(np.median(enum_ms)),
                            "output_voxels": int(ijk_out.shape[0]), "output_leaves": int(out.leaf_count)}
    return ops


def pyramid(binding, torch, np, synth, reps=20):
    """Workload 4 (16 res-64 shells): the encoder pyramid (coarsen x2 three
    times, 64 -> 32 -> 16 -> 8) and the decoder chain back up (k3s2 transpose
    three times from the coarsest level), each level built from the previous
    one on the GPU, timed as one rebuild (median of `reps`); the same rebuild
    with the kernel maps a plan pyramid needs (k3 s1 on each encoder level, the
    k2s2 conv map of each coarsening, the k3s2 transposed map of each decoder
    step); and single calls of refine / coarsen by 4 and 8 (PR page
    Measurements: the 4-level plan-pyramid row; section 1: factors 4 and 8)."""
    ijk, off = synth.make_config(4)
    src = binding.tc_batch_from_ijk(torch.from_numpy(ijk).cuda(), off)
    torch.cuda.synchronize()

    def rebuild(with_maps):
        enc = [src]
        for _ in range(3):
            enc.append(binding.tc_build_batched_topology(enc[-1], "coarsen", 2))
        dec = [enc[-1]]
        for _ in range(3):
            dec.append(binding.tc_build_batched_topology(dec[-1], "conv_t_k3s2", 2))
        maps = []
        if with_maps:
            for lvl in enc:
                maps.append(binding.tc_build_kernel_map(lvl, lvl, 3, 1, False))
            for a, b in zip(enc[:-1], enc[1:]):
                maps.append(binding.tc_build_kernel_map(a, b, 2, 2, False))
            for a, b in zip(dec[:-1], dec[1:]):
                maps.append(binding.tc_build_kernel_map(a, b, 3, 2, True))
        return enc, dec, maps

    res = {"workload": synth.CONFIG_NAMES[4], "grids": int(len(off) - 1), "input_voxels": int(off[-1])}
    for key, with_maps in [("rebuild_topology", False), ("rebuild_with_kernel_maps", True)]:
        rebuild(with_maps)  # warm-up
        ms = []
        for _ in range(reps):
            torch.cuda.synchronize()
            a = time.perf_counter()
            enc, dec, maps = rebuild(with_maps)
            torch.cuda.synchronize()
            ms.append((time.perf_counter() - a) * 1e3)
        res[key] = {"ms_median": float(np.median(ms)), "passes": 3 + 2 * 3, "kernel_maps": len(maps),
                    "level_voxels": [int(b.voxel_total()) for b in enc + dec[1:]],
                    "kernel_map_entries": int(sum(m.numel() for m in maps))}
        del enc, dec, maps
    singles = {}
    for op, f in [("refine", 4), ("refine", 8), ("coarsen", 4), ("coarsen", 8)]:
        binding.tc_build_batched_topology(src, op, f)  # warm-up
        ms = []
        for _ in range(reps):
            torch.cuda.synchronize()
            a = time.perf_counter()
            out = binding.tc_build_batched_topology(src, op, f)
            torch.cuda.synchronize()
            ms.append((time.perf_counter() - a) * 1e3)
        singles[f"{op}x{f}"] = {"ms_median": float(np.median(ms)), "passes": f.bit_length() - 1,
                                "output_voxels": int(out.voxel_total()), "output_leaves": int(out.leaf_count)}
        del out
    res["single_calls"] = singles
    return res


def cpu_baseline(np, ijk, off, large_input=None, min_s=10.0):
    """The CPU oracle (test infrastructure, untouched) on the host: whole steps of
    the workload with its members spread over the host's threads (>= min_s
    seconds), one step on one thread, and, when given, coarsen x2 of the
    46M-voxel batch on the host's threads."""
    import oracle
    threads = oracle.host_threads()
    t = time.perf_counter()
    cv, reps = 0, 0
    while True:
        for op, f in STEP_OPS:
            r = oracle.run_threaded(op, f, ijk, off, threads=threads, fields=["headers"])
            cv += int(r["headers"][:, 8].sum())
        reps += 1
        if time.perf_counter() - t >= min_s or reps >= 200:
            break
    dt = time.perf_counter() - t
    t1 = time.perf_counter()
    cv1 = 0
    for op, f in STEP_OPS:
        cv1 += int(oracle.run(op, f, ijk, off, fields=["headers"])["headers"][:, 8].sum())
    dt1 = time.perf_counter() - t1
    res = {"value": cv / dt, "unit": "voxels/s", "cores": threads, "kind": "oracle",
           "sample": f"{reps} full step(s) of the bench workload (all members, {len(STEP_OPS)} ops), {dt:.1f} s, "
                     f"members spread over {threads} host threads",
           "single_thread": {"value": cv1 / dt1, "unit": "voxels/s", "cores": 1,
                             "sample": f"one full step, {dt1:.1f} s"}}
    if large_input is not None:
        lijk, loff = large_input
        t2 = time.perf_counter()
        r = oracle.run_threaded("coarsen", 2, lijk, loff, threads=threads, fields=["headers"])
        dt2 = time.perf_counter() - t2
        res["shells512_cubes_coarsenx2"] = {"value": float(r["headers"][:, 8].sum()) / dt2, "unit": "voxels/s",
                                            "cores": threads, "seconds": dt2,
                                            "sample": "coarsen x2 of all 72 members of the 46M-voxel batch"}
    return res


def progress(msg):
    """A progress line on stderr (the JSON result is the only stdout line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def run_step(binding, src, outs=None, one_call=True, allocator="none"):
    """One step: every op's target, then each target's voxel enumeration. With
    `one_call` the targets come from one tc_build_batched_topology_many call and
    their enumerations from one tc_enumerate_ijk_many launch, else from one
    tc_build_batched_topology and one tc_enumerate_ijk call per op. `allocator`
    "none" takes the outputs from the library's own stream-ordered pool (the C
    ABI's default, a NULL allocator), "torch" from torch's caching allocator
    through the binding's callback. Returns voxels."""
    total = 0
    if one_call:
        built = binding.tc_build_batched_topology_many(src, STEP_OPS, allocator=allocator)
    else:
        built = [binding.tc_build_batched_topology(src, op, f, allocator=allocator) for op, f in STEP_OPS]
    if one_call:
        ijks = binding.tc_enumerate_ijk_many(built)
    else:
        ijks = [binding.tc_enumerate_ijk(out) for out in built]
    for (op, f), out, ijk in zip(STEP_OPS, built, ijks):
        total += ijk.shape[0]
        if outs is not None:
            outs.append((op, f, out.leaf_count, int(ijk.shape[0])))
    return total


# Algorithmic bytes of one launch of each measured kernel: what the step itself
# must move, not what the kernel happens to move.
#   k_leaf_mark_*        reads every source leaf once: origin 16 B + mask 64 B
#                        (k_leaf_mark_lower: refine / coarsen; k_leaf_mark_box: box ops)
#   k_leaf_gather        reads every output leaf's origin 16 B + candidate id 4 B, every
#                        source mask once (64 B), writes every output mask (64 B)
#   k_leaf_offsets_bbox  reads origin 16 B + packed bbox 4 B + voxel scan 8 B,
#                        writes the voxel offset 8 B, per output leaf (k_finalize_small,
#                        the same work in one launch on batches of at most 262144 leaves)
#   k_enumerate          reads origin, mask, offset and grid base (96 B per leaf),
#                        writes 12 B per voxel
def kernel_bytes(name, src_leaves, leaves, voxels):
    if name in ("k_leaf_mark_lower", "k_leaf_mark_box"):
        return 80 * src_leaves
    if name == "k_leaf_gather":
        return 84 * leaves + 64 * src_leaves
    if name in ("k_leaf_offsets_bbox", "k_finalize_small"):
        return 36 * leaves
    if name == "k_enumerate":
        return 96 * leaves + 12 * voxels
    raise ValueError(name)


LARGE_KERNELS = ["k_leaf_mark_lower", "k_leaf_mark_box", "k_leaf_gather", "k_leaf_offsets_bbox", "k_finalize_small",
                 "k_enumerate"]


def source_digest():
    """sha256 over the library's kernel sources with // comments, trailing blanks
    and empty lines removed: counter readings taken from other code no longer
    describe the kernels and are then not reported (a comment edit changes no
    kernel, so it keeps them)."""
    csrc = os.path.join(ROOT, "topology_construction_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp")):
            with open(os.path.join(csrc, name), encoding="utf-8") as fh:
                lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in fh]
            h.update(name.encode() + b"\0" + "\n".join(ln for ln in lines if ln).encode())
    return h.hexdigest()


def recorded_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed counter summary
    profiles/traffic_<kernel>_<workload>.txt (lines `key value`), or None when
    there is none or it was taken from other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            parts = line.split()
            if len(parts) == 2:
                kv[parts[0]] = parts[1]
    if kv.get("source_sha256") != source_digest() or "hbm_bytes_per_launch" not in kv:
        return None
    return float(kv["hbm_bytes_per_launch"])


def recorded_trace_ms(kernel, workload):
    """Average kernel-trace duration (ms) of `kernel` over the bench's timed
    launches, from the committed summary profiles/trace_<kernel>_<workload>.txt
    (lines `key value`), or None when there is none or it was taken from other
    kernel sources."""
    path = os.path.join(ROOT, "profiles", f"trace_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            parts = line.split()
            if len(parts) == 2 and not line.startswith("#"):
                kv[parts[0]] = parts[1]
    if kv.get("source_sha256") != source_digest() or "trace_avg_us_timed" not in kv:
        return None
    return float(kv["trace_avg_us_timed"]) * 1e-3


def copy_calibration(torch, mib):
    """Three device-to-device copies of `mib` MiB (reads and writes mib MiB each)."""
    if mib <= 0:
        return
    a = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()


def time_from_ijk(binding, torch, np, d_ijk, off, reps):
    """The ijk front-end on device-resident rows: median wall ms and its rate.
    Algorithmic bytes: 12 B read per input voxel, 100 B written per output leaf
    (origin, mask, prefix, offset, parent)."""
    ms, leaves = [], 0
    for _ in range(reps):
        torch.cuda.synchronize()
        a = time.perf_counter()
        b = binding.tc_batch_from_ijk(d_ijk, off)
        torch.cuda.synchronize()
        ms.append((time.perf_counter() - a) * 1e3)
        leaves = int(b.leaf_count)
        del b
    m = float(np.median(ms))
    n = int(off[-1])
    byts = 12 * n + 100 * leaves
    return {"ms_median": m, "input_voxels": n, "output_leaves": leaves, "input_voxels_per_s": n / (m * 1e-3),
            "algorithmic_bytes": byts, "achieved_GBs": byts / (m * 1e-3) / 1e9}


def time_from_points(binding, torch, np, d_ijk, off, reps):
    """The points front-end (mode 0, voxel size 1, origin 0) on device-resident
    float32 points a quarter voxel off the centres: median wall ms and its rate."""
    B = len(off) - 1
    pts = d_ijk.to(torch.float32) + 0.25
    vs, org = np.ones((B, 3), np.float32), np.zeros((B, 3), np.float32)
    ms, leaves = [], 0
    binding.tc_batch_from_points(pts, off, vs, org, 0)  # warm-up
    for _ in range(reps):
        torch.cuda.synchronize()
        a = time.perf_counter()
        b = binding.tc_batch_from_points(pts, off, vs, org, 0)
        torch.cuda.synchronize()
        ms.append((time.perf_counter() - a) * 1e3)
        leaves = int(b.leaf_count)
        del b
    m = float(np.median(ms))
    n = int(off[-1])
    return {"ms_median": m, "input_points": n, "output_leaves": leaves, "input_points_per_s": n / (m * 1e-3)}


def time_kernel_maps(binding, torch, np, src, reps):
    """The two kernel maps a plan builds (issue page, Measurements): k3 s1 on the
    source's own topology and k2s2 transposed conv onto refine x2. Output tables
    are allocated once, outside the timing. Algorithmic bytes of one
    k_kernel_map launch: the table it writes (4 B per entry) plus one read of
    every target leaf (origin, mask, offset: 88 B) and source leaf (mask,
    prefix, offset: 80 B)."""
    fine = binding.tc_build_batched_topology(src, "refine", 2)
    res = {}
    for name, dst, k, s, t in [("k3s1_same_topology", src, 3, 1, False), ("k2s2_transposed_onto_refine", fine, 2, 2, True)]:
        rows = dst.voxel_total()
        out = torch.empty((rows, k ** 3), dtype=torch.int32, device="cuda")
        binding.tc_build_kernel_map(src, dst, k, s, t, out=out)  # warm-up
        torch.cuda.synchronize()
        binding.tc_profile_enable("k_kernel_map")
        ms = []
        for _ in range(reps):
            torch.cuda.synchronize()
            a = time.perf_counter()
            binding.tc_build_kernel_map(src, dst, k, s, t, out=out)
            torch.cuda.synchronize()
            ms.append((time.perf_counter() - a) * 1e3)
        k_ms, k_n = binding.tc_profile_read("k_kernel_map")
        binding.tc_profile_disable()
        entries = rows * k ** 3
        byts = 4 * entries + 88 * int(dst.leaf_count) + 80 * int(src.leaf_count)
        avg = k_ms / max(k_n, 1)
        res[name] = {"ms_median": float(np.median(ms)), "kernel_avg_ms": avg, "rows": int(rows),
                     "entries": int(entries), "valid_entries": int((out >= 0).sum().item()),
                     "algorithmic_bytes": byts, "achieved_GBs": byts / (avg * 1e-3) / 1e9,
                     "frac_of_peak": byts / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del out
    del fine
    return res


def measure_large(binding, torch, np, synth, keep_input=None):
    """64 shells at res 512 + 8 solid 128^3 cubes: per-op pass / enumeration time
    and per-kernel HIP-event timing against the HBM peak. `keep_input`, a list,
    receives the host input (ijk, offsets) for the CPU baseline."""
    ijk, off = synth.make_config(5)
    d_ijk = torch.from_numpy(ijk).cuda()
    if keep_input is not None:
        keep_input.append((ijk, off))
    del ijk
    src = binding.tc_batch_from_ijk(d_ijk, off)
    torch.cuda.synchronize()
    res = {"workload": synth.CONFIG_NAMES[5], "grids": int(len(off) - 1), "input_voxels": int(off[-1]),
           "input_leaves": int(src.leaf_count), "from_ijk": time_from_ijk(binding, torch, np, d_ijk, off, 3),
           "from_points": time_from_points(binding, torch, np, d_ijk, off, 3), "ops": {}}
    del d_ijk
    for op, f in [("coarsen", 2), ("refine", 2), ("dilate", 1)]:
        out = binding.tc_build_batched_topology(src, op, f)  # warm-up
        binding.tc_enumerate_ijk(out)
        del out
        torch.cuda.synchronize()
        binding.tc_profile_enable(",".join(LARGE_KERNELS))
        pass_ms, enum_ms = [], []
        for _ in range(3):
            torch.cuda.synchronize()
            a = time.perf_counter()
            out = binding.tc_build_batched_topology(src, op, f)
            torch.cuda.synchronize()
            b = time.perf_counter()
            e = binding.tc_enumerate_ijk(out)
            torch.cuda.synchronize()
            c = time.perf_counter()
            pass_ms.append((b - a) * 1e3)
            enum_ms.append((c - b) * 1e3)
            V = int(e.shape[0])
            L = int(out.leaf_count)
            del e, out
        kern = {}
        for k in LARGE_KERNELS:
            ms, n = binding.tc_profile_read(k)
            if n:
                avg = ms / n
                byts = kernel_bytes(k, int(src.leaf_count), L, V)
                gbs = byts / (avg * 1e-3) / 1e9
                kern[k] = {"avg_ms": avg, "launches": n, "algorithmic_bytes": byts, "achieved_GBs": gbs,
                           "frac_of_peak": gbs / HBM_PEAK_GBS}
        binding.tc_profile_disable()
        pm = float(np.median(pass_ms))
        progress(f"large {op}x{f} done")
        res["ops"][f"{op}x{f}"] = {"ms_pass_median": pm, "ms_enumerate_median": float(np.median(enum_ms)),
                                   "output_voxels": V, "output_leaves": L,
                                   "output_voxels_per_s_pass": V / (pm * 1e-3), "kernels": kern}
    res["kernel_maps"] = time_kernel_maps(binding, torch, np, src, 3)
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; run with --gpus 1"}))
        sys.exit(2)
    import numpy as np
    import torch

    from topology_construction_amd import binding, synth

    torch.cuda.set_device(0)
    if args.large_only:
        print(json.dumps({"large": measure_large(binding, torch, np, synth)}), flush=True)
        copy_calibration(torch, args.copy_mib)
        return
    ijk, off = synth.make_config(args.config)
    d_ijk = torch.from_numpy(ijk).cuda()
    src = binding.tc_batch_from_ijk(d_ijk, off)
    torch.cuda.synchronize()

    # per-op launch facts for the roofline bytes
    facts = []
    run_step(binding, src, facts)
    for _ in range(args.warmup):
        run_step(binding, src)
    torch.cuda.synchronize()

    binding.tc_profile_enable(args.roofline_kernel)
    t0 = time.perf_counter()
    voxels = 0
    for _ in range(args.steps):
        voxels += run_step(binding, src)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    k_ms, k_n = binding.tc_profile_read(args.roofline_kernel)
    binding.tc_profile_disable()
    elapsed = t1 - t0
    ms_step = elapsed * 1e3 / args.steps
    # the same steps without the timing events (their cost, beside the headline)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(args.steps):
        run_step(binding, src)
    torch.cuda.synchronize()
    ms_step_plain = (time.perf_counter() - t2) * 1e3 / args.steps
    # the same steps with one build call per op (each waits for its own headers)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(args.steps):
        run_step(binding, src, one_call=False)
    torch.cuda.synchronize()
    ms_step_single = (time.perf_counter() - t2) * 1e3 / args.steps
    # and with torch's caching allocator supplying the outputs (a ctypes callback each)
    for _ in range(args.warmup):
        run_step(binding, src, allocator="torch")
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(args.steps):
        run_step(binding, src, allocator="torch")
    torch.cuda.synchronize()
    ms_step_torch = (time.perf_counter() - t2) * 1e3 / args.steps

    # per-op breakdown (separate, untimed-by-the-step loop): pass and enumeration
    progress(f"timed steps done: {ms_step:.4f} ms per step")
    ops = op_medians(binding, torch, np, src)
    progress("per-op medians, 16 shells, done")
    # the same at B=48 (mixed member sizes, three empty members, members
    # straddling +-4096 tiles): how flat the batched pass stays as B triples
    ijk48, off48 = synth.make_config(3)
    src48 = binding.tc_batch_from_ijk(torch.from_numpy(ijk48).cuda(), off48)
    ops48 = op_medians(binding, torch, np, src48)
    progress("per-op medians, 48 shells, done")
    b48 = {"workload": synth.CONFIG_NAMES[3], "grids": int(len(off48) - 1), "input_voxels": int(off48[-1]),
           "ops": ops48,
           "pass_ratio_b48_over_b16": {k: ops48[k]["ms_pass_median"] / ops[k]["ms_pass_median"] for k in ops}}
    del src48
    # B=2 (resolution 16): the smallest batch, for the flatness in B
    ijk2, off2 = synth.make_config(1)
    src2 = binding.tc_batch_from_ijk(torch.from_numpy(ijk2).cuda(), off2)
    b2 = {"workload": synth.CONFIG_NAMES[1], "grids": int(len(off2) - 1), "input_voxels": int(off2[-1]),
          "ops": op_medians(binding, torch, np, src2)}
    del src2
    pyr = pyramid(binding, torch, np, synth)
    progress("pyramid done")

    # the rows beyond the step: stride-1 kernel-K targets and masked refine (60% kept)
    gen = torch.Generator(device="cuda").manual_seed(11)
    keep = (torch.rand(src.voxel_total(), device="cuda", generator=gen) < 0.6).to(torch.uint8)
    extra_ops = [("conv_s1", 2), ("conv_s1", 4), ("conv_s1", 5), ("conv_t_s1", 2), ("conv_t_s1", 4), ("masked_refine", 2)]
    extra = {}
    for op, f in extra_ops:
        pass_ms = []
        for _ in range(20):
            torch.cuda.synchronize()
            a = time.perf_counter()
            if op == "masked_refine":
                out = binding.tc_build_masked_refine(src, keep, f)
            else:
                out = binding.tc_build_batched_topology(src, op, f)
            torch.cuda.synchronize()
            pass_ms.append((time.perf_counter() - a) * 1e3)
        extra[f"{op}x{f}"] = {"ms_median": float(np.median(pass_ms)), "output_voxels": int(out.voxel_total()),
                              "output_leaves": int(out.leaf_count)}
        del out

    bytes_per_step = sum(kernel_bytes(args.roofline_kernel, int(src.leaf_count), L, V) for (_, _, L, V) in facts)
    # launches of the kernel per step, as the timed steps made them (one batched
    # enumeration per step; a per-op kernel would launch once per op)
    launches_per_step = k_n / args.steps if k_n else len(facts)
    avg_ms = k_ms / max(k_n, 1)
    avg_bytes = bytes_per_step / launches_per_step
    achieved = avg_bytes / (avg_ms * 1e-3) / 1e9 if k_n else None
    tag = WORKLOAD_TAGS.get(args.config, f"config{args.config}")
    roofline = {"bound": "hbm", "kernel": args.roofline_kernel, "achieved": achieved, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": (achieved / HBM_PEAK_GBS) if achieved else None,
                "traffic": recorded_traffic(args.roofline_kernel, tag),
                "avg_launch_ms": avg_ms, "launches": k_n, "algorithmic_bytes_per_launch": avg_bytes}
    trace_ms = recorded_trace_ms(args.roofline_kernel, tag)
    if trace_ms:
        # the kernel's own duration in the rocprofv3 trace of the same timed
        # launches (the events above also hold each launch's dispatch)
        roofline["trace_avg_launch_ms"] = trace_ms
        roofline["achieved_trace"] = avg_bytes / (trace_ms * 1e-3) / 1e9
        roofline["frac_trace"] = roofline["achieved_trace"] / HBM_PEAK_GBS

    large_input = []
    progress("extra ops done")
    large = None if args.no_large else measure_large(binding, torch, np, synth, keep_input=large_input)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(np, ijk, off, large_input[0] if large_input else None)

    rec = {
        "metric": METRIC, "value": voxels / elapsed, "unit": "voxels/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "ms_per_step_unprofiled": ms_step_plain,
        "ms_per_step_one_call_per_op": ms_step_single, "ms_per_step_torch_allocator": ms_step_torch,
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int32", "data": "synthetic",
        "config": {"workload": synth.CONFIG_NAMES[args.config], "grids": int(len(off) - 1),
                   "input_voxels": int(off[-1]), "ops": [f"{o}x{f}" for o, f in STEP_OPS]},
        "roofline": roofline, "cpu_baseline": cpu, "ops": ops, "b48": b48, "b2": b2, "pyramid": pyr,
        "more_ops": extra,
        "from_ijk": time_from_ijk(binding, torch, np, d_ijk, off, 20),
        "from_points": time_from_points(binding, torch, np, d_ijk, off, 20),
        "kernel_maps": time_kernel_maps(binding, torch, np, src, 20), "large": large,
    }
    print(json.dumps(rec), flush=True)
    copy_calibration(torch, args.copy_mib)


if __name__ == "__main__":
    main()
