"""Seeded synthetic voxel-grid batches (ellipsoid shells and solid cubes).

This module only draws inputs. It holds none of the topology arithmetic
(coarsen / refine / dilate / ordering), so both the HIP path and the CPU
oracle can consume the very same int32 arrays it returns.

Workload shapes follow the batched-topology PR page ("Batched leaf-mask topology
construction for generated conv grids", Measurements section): synthetic shell
batches of about 7.8k voxels per member at resolution 64, B = 16 and 48.

Shell membership test (first-order distance to an axis-aligned ellipsoid):
with q = p + 0.5 - c, rho = |q / r| and g = |q / r^2| / rho, voxel p is kept when
|rho - 1| < 0.5 * g, i.e. the estimated distance to the surface is under half a
voxel. The test is evaluated only on a narrow band of candidate voxels per
(x, y) column; the band is a superset of the kept set because g <= 1 / min(r).

Every array is int32 [N, 3] with int64 offsets [B + 1]; members are concatenated
in order and an empty member has offsets[g] == offsets[g + 1].
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "shell_voxels",
    "shell_voxels_bruteforce",
    "cube_voxels",
    "concat_members",
    "make_config",
    "CONFIG_NAMES",
]

CONFIG_NAMES = {
    1: "shells B=2 res16",
    2: "shells B=16 res64",
    3: "mixed shells B=48 res64 (3 empty, translated, tile-straddling)",
    4: "pyramid shells B=16 res64",
    5: "64 shells res512 + 8 solid 128^3 cubes",
}


def _keep(px, py, pz, c, r):
    qx = px + 0.5 - c[0]
    qy = py + 0.5 - c[1]
    qz = pz + 0.5 - c[2]
    ax, ay, az = qx / r[0], qy / r[1], qz / r[2]
    rho = np.sqrt(ax * ax + ay * ay + az * az)
    bx, by, bz = ax / r[0], ay / r[1], az / r[2]
    gnorm = np.sqrt(bx * bx + by * by + bz * bz)
    with np.errstate(divide="ignore", invalid="ignore"):
        g = gnorm / rho
        keep = np.abs(rho - 1.0) < 0.5 * g
    return keep & (rho > 0)


def shell_voxels_bruteforce(res: int, center, radii) -> np.ndarray:
    """Evaluate the shell test on every voxel of [0, res)^3 (small res only)."""
    c = np.asarray(center, dtype=np.float64)
    r = np.asarray(radii, dtype=np.float64)
    g = np.arange(res, dtype=np.float64)
    px, py, pz = np.meshgrid(g, g, g, indexing="ij")
    k = _keep(px, py, pz, c, r)
    idx = np.nonzero(k)
    return np.stack(idx, axis=1).astype(np.int32)


def shell_voxels(res: int, center, radii) -> np.ndarray:
    """Narrow-band evaluation of the shell test; same set as the brute force.

    Output order: x-major, then y, then z ascending within each column.
    """
    c = np.asarray(center, dtype=np.float64)
    r = np.asarray(radii, dtype=np.float64)
    delta = 0.5 / float(r.min())
    g = np.arange(res, dtype=np.float64)
    X, Y = np.meshgrid(g, g, indexing="ij")
    X = X.ravel()
    Y = Y.ravel()
    tx = (X + 0.5 - c[0]) / r[0]
    ty = (Y + 0.5 - c[1]) / r[1]
    t = tx * tx + ty * ty
    hi2 = (1.0 + delta) ** 2 - t
    lo2 = np.maximum((1.0 - delta) ** 2 - t, 0.0)
    live = hi2 >= 0
    X, Y, hi2, lo2 = X[live], Y[live], hi2[live], lo2[live]
    A = r[2] * np.sqrt(hi2)
    a = r[2] * np.sqrt(lo2)
    # two z intervals per column: qz in [-A, -a] and [a, A]; z = qz + c_z - 0.5
    zc = c[2] - 0.5
    iv = []
    for lo, hi in ((-A + zc, -a + zc), (a + zc, A + zc)):
        zl = np.clip(np.floor(lo) - 1, 0, res - 1).astype(np.int64)
        zh = np.clip(np.ceil(hi) + 1, 0, res - 1).astype(np.int64)
        iv.append((zl, zh))
    # merge overlapping intervals so no candidate is tested twice
    (l0, h0), (l1, h1) = iv
    overlap = l1 <= h0 + 1
    h0m = np.where(overlap, np.maximum(h0, h1), h0)
    l1m = np.where(overlap, 1, l1)
    h1m = np.where(overlap, 0, h1)  # empty second interval
    xs, ys, zs = [], [], []
    for lo, hi in ((l0, h0m), (l1m, h1m)):
        n = np.maximum(hi - lo + 1, 0)
        tot = int(n.sum())
        if tot == 0:
            continue
        colx = np.repeat(X, n)
        coly = np.repeat(Y, n)
        start = np.repeat(lo, n)
        first = np.repeat(np.cumsum(n) - n, n)
        z = start + (np.arange(tot, dtype=np.int64) - first)
        xs.append(colx)
        ys.append(coly)
        zs.append(z.astype(np.float64))
    if not xs:
        return np.zeros((0, 3), dtype=np.int32)
    px = np.concatenate(xs)
    py = np.concatenate(ys)
    pz = np.concatenate(zs)
    k = _keep(px, py, pz, c, r)
    out = np.stack([px[k], py[k], pz[k]], axis=1).astype(np.int64)
    order = np.lexsort((out[:, 2], out[:, 1], out[:, 0]))
    return out[order].astype(np.int32)


def cube_voxels(side: int, offset) -> np.ndarray:
    g = np.arange(side, dtype=np.int64)
    X, Y, Z = np.meshgrid(g, g, g, indexing="ij")
    v = np.stack([X.ravel(), Y.ravel(), Z.ravel()], axis=1) + np.asarray(offset, dtype=np.int64)
    return v.astype(np.int32)


def concat_members(members):
    counts = [int(m.shape[0]) for m in members]
    offsets = np.zeros(len(members) + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    if offsets[-1] == 0:
        return np.zeros((0, 3), dtype=np.int32), offsets
    ijk = np.concatenate([m.reshape(-1, 3) for m in members], axis=0).astype(np.int32)
    return np.ascontiguousarray(ijk), offsets


def _shell_member(rng, res, lo, hi):
    radii = rng.uniform(lo, hi, size=3) * res
    center = rng.uniform(0.45, 0.55, size=3) * res
    return shell_voxels(res, center, radii)


def make_config(cfg: int, seed: int | None = None):
    """Return (ijk int32 [N,3], offsets int64 [B+1]) for workload `cfg` (1..5).

    1: B=2 shells at res 16, radii U[0.3,0.45]*res, centre U[0.45,0.55]*res.
    2: B=16 shells at res 64 (same radius range).
    3: B=48 shells at res 64 with radius scale U[0.1,0.45]; members 0, 24, 47 empty;
       odd members translated by U_int[-4200,4200]^3, with members 1, 3, 5 forced to
       (-4128)^3, (-32)^3 and (4064)^3 so that they straddle the -4096, 0 and +4096
       root-tile boundaries on every axis.
    4: B=16 shells at res 64 (the pyramid workload's base level).
    5: 64 shells at res 512 plus 8 solid 128^3 cubes at offsets U_int[-2^29, 2^29)^3.
    """
    if seed is None:
        seed = cfg
    rng = np.random.default_rng(seed)
    members = []
    if cfg == 1:
        for _ in range(2):
            members.append(_shell_member(rng, 16, 0.3, 0.45))
    elif cfg in (2, 4):
        for _ in range(16):
            members.append(_shell_member(rng, 64, 0.3, 0.45))
    elif cfg == 3:
        empty = {0, 24, 47}
        forced = {1: -4128, 3: -32, 5: 4064}
        for g in range(48):
            m = _shell_member(rng, 64, 0.1, 0.45)
            off = rng.integers(-4200, 4201, size=3)
            if g in empty:
                m = m[:0]
            elif g % 2 == 1:
                if g in forced:
                    off = np.full(3, forced[g], dtype=np.int64)
                m = (m.astype(np.int64) + off).astype(np.int32)
            members.append(m)
    elif cfg == 5:
        for _ in range(64):
            members.append(_shell_member(rng, 512, 0.3, 0.45))
        for _ in range(8):
            off = rng.integers(-(1 << 29), 1 << 29, size=3)
            members.append(cube_voxels(128, off))
    else:
        raise ValueError(f"unknown workload {cfg}")
    return concat_members(members)
