"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
bring every output array to numpy in the oracle's layout."""
import numpy as np

import oracle
from topology_construction_amd import binding

HEADER_COLS = oracle.HEADER_COLUMNS


def headers_as_oracle(h: np.ndarray) -> np.ndarray:
    """Structured tc_grid_header[B] -> int64 [B, 16] in the oracle's column order."""
    out = np.zeros((h.shape[0], 16), dtype=np.int64)
    for k, name in enumerate(HEADER_COLS[:10]):
        out[:, k] = h[name]
    out[:, 10:13] = h["bbox_min"]
    out[:, 13:16] = h["bbox_max"]
    return out


def gpu_fields(batch: binding.GridBatch) -> dict:
    import torch
    torch.cuda.synchronize()
    out = {}
    for name, t in batch.fields().items():
        a = t.cpu().numpy()
        out[name] = a
    out["headers"] = headers_as_oracle(batch.headers())
    out["ijk"] = batch.ijk().cpu().numpy()
    torch.cuda.synchronize()
    return out


def gpu_build(op: str, factor: int, ijk: np.ndarray, offsets: np.ndarray, src=None):
    """from_ijk (and the op unless op == 'identity') on the GPU; returns (batch, src)."""
    import torch
    if src is None:
        t = torch.from_numpy(np.ascontiguousarray(ijk, dtype=np.int32).reshape(-1, 3)).cuda()
        src = binding.tc_batch_from_ijk(t, offsets)
    if op == "identity":
        return src, src
    return binding.tc_build_batched_topology(src, op, factor), src


def assert_same(gpu: dict, ref: dict, ctx=""):
    for name in oracle.FIELDS:
        g, r = gpu[name], ref[name]
        assert g.shape == r.shape, f"{ctx} {name}: shape {g.shape} vs oracle {r.shape}"
        if not np.array_equal(g, r):
            bad = np.argwhere(g != r)
            raise AssertionError(f"{ctx} {name}: {bad.shape[0]} mismatches, first at {bad[:3].tolist()}; "
                                 f"gpu {g[tuple(bad[0])]} oracle {r[tuple(bad[0])]}")


def member_slice(f: dict, g: int) -> dict:
    """Member g of a batch in single-member form (indices rebased, grid id 0)."""
    h = f["headers"][g]
    nu, n1, nl, ub, lb, leafb, nv, vb = (int(h[k]) for k in (2, 3, 4, 5, 6, 7, 8, 9))
    out = {}
    uo = f["upper_origin"][ub:ub + nu].copy()
    uo[:, 3] = 0
    out["upper_origin"] = uo
    out["upper_key"] = f["upper_key"][ub:ub + nu]
    out["upper_first"] = f["upper_first"][ub:ub + nu] - lb
    out["upper_mask"] = f["upper_mask"][ub:ub + nu]
    lo = f["lower_origin"][lb:lb + n1].copy()
    lo[:, 3] -= ub
    out["lower_origin"] = lo
    out["lower_first"] = f["lower_first"][lb:lb + n1] - leafb
    out["lower_mask"] = f["lower_mask"][lb:lb + n1]
    out["lower_prefix"] = f["lower_prefix"][lb:lb + n1]
    lf = f["leaf_origin"][leafb:leafb + nl].copy()
    lf[:, 3] = 0
    out["leaf_origin"] = lf
    out["leaf_parent"] = f["leaf_parent"][leafb:leafb + nl] - lb
    out["leaf_mask"] = f["leaf_mask"][leafb:leafb + nl]
    out["leaf_prefix"] = f["leaf_prefix"][leafb:leafb + nl]
    out["leaf_offset"] = f["leaf_offset"][leafb:leafb + nl]
    out["ijk"] = f["ijk"][vb:vb + nv]
    hh = h.copy()
    hh[0] = 0
    hh[1] = 1
    hh[5:8] = 0
    hh[9] = 0
    out["headers"] = hh[None, :]
    return out
