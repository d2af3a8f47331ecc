"""Oracle point-cloud voxelisation (test infrastructure only; see the package docstring).

spconv's ``PointToVoxel`` (spconv USAGE.md, "spconv.pytorch.utils API
Reference" and "Converting Point Clouds to Voxels using
spconv.pytorch.utils.PointToVoxel"): points ``[N, F]`` (x, y, z first) fall
into voxels of size ``vsize_xyz`` over the box ``coors_range_xyz``; the
result is up to ``max_num_voxels`` voxels of up to
``max_num_points_per_voxel`` points each, their ZYX integer coordinates (no
batch axis), their point counts, and for every point the id of the voxel
that holds it (or -1: outside the box, or no room).  With ``empty_mean`` the
unused point slots of a voxel hold the mean of its points, else zeros.
``gather_features_by_pc_voxel_id`` reads per-voxel features back per point,
zeros for id -1.

Readings where the pages are silent:

* grid extent per axis: ``round((max - min) / vsize)`` (in float64 of the
  float32 arguments, half to even);
* voxel coordinate: ``floor((p - min) / vsize)`` in float32 (each operation
  rounded to nearest); a point is inside iff ``0 <= c < extent`` on all axes;
* voxel ids number the voxels in order of their first point;
* a voxel keeps its first points in point order; once ``max_num_voxels``
  voxels exist, points of any further voxel are dropped;
* a point that is not stored (outside, or no room) has id -1;
* the mean of ``empty_mean`` is over the stored points, all F features.

The function below is the plain sequential loop over the points in order,
which is exactly that definition.
"""

from __future__ import annotations

import numpy as np


def grid_extent(vsize_xyz, range_xyz) -> np.ndarray:
    """Voxels per axis (x, y, z): ``round((max - min) / vsize)``."""
    v = np.asarray(vsize_xyz, np.float32).astype(np.float64)
    r = np.asarray(range_xyz, np.float32).astype(np.float64)
    return np.round((r[3:] - r[:3]) / v).astype(np.int64)


def voxel_coords(points, vsize_xyz, range_xyz):
    """Per point: integer (x, y, z) voxel coordinates (float32 arithmetic) and
    whether the point lies inside the grid."""
    p = np.asarray(points, np.float32)[:, :3]
    v = np.asarray(vsize_xyz, np.float32)
    lo = np.asarray(range_xyz, np.float32)[:3]
    with np.errstate(invalid="ignore"):
        c = np.floor((p - lo) / v)  # float32 throughout
        inside = np.all((c >= 0) & (c < grid_extent(vsize_xyz, range_xyz)), axis=1)
    return np.where(inside[:, None], c, 0).astype(np.int64), inside


def point_to_voxel(points, vsize_xyz, range_xyz, max_voxels: int, max_points: int, empty_mean: bool = True):
    """``(voxels [V, max_points, F] f32, coords [V, 3] int32 (z, y, x),
    num_points [V] int32, pc_voxel_id [N] int32)`` by one pass over the points."""
    pts = np.asarray(points, np.float32)
    N, F = pts.shape
    c, inside = voxel_coords(pts, vsize_xyz, range_xyz)
    ids = {}
    voxels, coords, counts = [], [], []
    pcid = np.full(N, -1, np.int32)
    for i in range(N):
        if not inside[i]:
            continue
        key = (int(c[i, 2]), int(c[i, 1]), int(c[i, 0]))  # z, y, x
        v = ids.get(key)
        if v is None:
            if len(voxels) >= max_voxels:
                continue
            v = ids[key] = len(voxels)
            voxels.append(np.zeros((max_points, F), np.float32))
            coords.append(key)
            counts.append(0)
        if counts[v] < max_points:
            voxels[v][counts[v]] = pts[i]
            counts[v] += 1
            pcid[i] = v
    for v, n in enumerate(counts):
        if empty_mean and n < max_points:
            voxels[v][n:] = (voxels[v][:n].astype(np.float64).sum(axis=0) / n).astype(np.float32)
    V = len(voxels)
    return (np.stack(voxels) if V else np.zeros((0, max_points, F), np.float32),
            np.asarray(coords, np.int32).reshape(V, 3), np.asarray(counts, np.int32), pcid)


def gather_by_voxel_id(seg_features, pc_voxel_id) -> np.ndarray:
    """``out[i] = seg_features[pc_voxel_id[i]]``, zeros where the id is -1."""
    f = np.asarray(seg_features)
    idx = np.asarray(pc_voxel_id)
    out = np.zeros((idx.shape[0],) + f.shape[1:], f.dtype)
    ok = idx >= 0
    out[ok] = f[idx[ok]]
    return out
