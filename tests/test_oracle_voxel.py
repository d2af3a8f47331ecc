"""Pins of the oracle's point-cloud voxelisation: a lattice with one point per
voxel (closed form), hand-built overflow of points and voxels, a second,
vectorised formulation of the same definition on random clouds, and the
invariants of the page's own example configuration."""

import numpy as np
import pytest

import workloads as W
from oracle import voxel as V

PAGE = dict(vsize_xyz=[0.1, 0.1, 0.1], range_xyz=[-80, -80, -2, 80, 80, 6])  # the USAGE.md example


def test_lattice_one_point_per_voxel():
    r = W.rng(200)
    zyx = np.stack(np.meshgrid(np.arange(3), np.arange(4), np.arange(5), indexing="ij"), -1).reshape(-1, 3)
    zyx = zyx[r.permutation(len(zyx))]
    xyz = (zyx[:, ::-1] + 0.5) * np.array([0.5, 0.25, 1.0]) + np.array([-1.0, 2.0, 0.0])
    pts = np.concatenate([xyz, r.standard_normal((len(zyx), 2))], 1).astype(np.float32)
    vox, coords, num, pcid = V.point_to_voxel(pts, [0.5, 0.25, 1.0], [-1, 2, 0, 1.5, 3, 3], 100, 4)
    np.testing.assert_array_equal(coords, zyx)              # first appearance = point order here
    np.testing.assert_array_equal(num, np.ones(len(zyx)))
    np.testing.assert_array_equal(pcid, np.arange(len(zyx)))
    np.testing.assert_array_equal(vox, np.repeat(pts[:, None], 4, 1))  # the mean of one point is the point


def test_overflow_of_points_and_voxels():
    pts = np.array([[0.5, 0.5, 0.5], [1.5, 0.5, 0.5], [0.2, 0.3, 0.4], [0.9, 0.9, 0.9], [2.5, 2.5, 2.5],
                    [1.1, 0.1, 0.1], [-0.1, 0.5, 0.5], [0.5, 0.5, 4.0]], np.float32)
    vox, coords, num, pcid = V.point_to_voxel(pts, [1, 1, 1], [0, 0, 0, 4, 4, 4], 2, 2, empty_mean=False)
    np.testing.assert_array_equal(coords, [[0, 0, 0], [0, 0, 1]])
    np.testing.assert_array_equal(num, [2, 2])
    np.testing.assert_array_equal(pcid, [0, 1, 0, -1, -1, 1, -1, -1])   # full voxel, no voxel left, outside x2
    np.testing.assert_array_equal(vox[0], pts[[0, 2]])
    np.testing.assert_array_equal(vox[1], pts[[1, 5]])
    vox, coords, num, pcid = V.point_to_voxel(pts, [1, 1, 1], [0, 0, 0, 4, 4, 4], 3, 3, empty_mean=True)
    np.testing.assert_array_equal(num, [3, 2, 1])
    np.testing.assert_array_equal(pcid, [0, 1, 0, 0, 2, 1, -1, -1])
    np.testing.assert_allclose(vox[1, 2], [1.3, 0.3, 0.3], rtol=1e-6)   # mean of points 1 and 5
    np.testing.assert_array_equal(vox[2], np.repeat(pts[[4]], 3, 0))
    vox0, *_ = V.point_to_voxel(pts, [1, 1, 1], [0, 0, 0, 4, 4, 4], 3, 3, empty_mean=False)
    np.testing.assert_array_equal(vox0[1, 2], [0, 0, 0])


def _vectorised(pts, vsize, rng_xyz, max_voxels, max_points, empty_mean):
    """The same definition through unique / first-index / stable-sort primitives."""
    c, inside = V.voxel_coords(pts, vsize, rng_xyz)
    ext = V.grid_extent(vsize, rng_xyz)
    key = np.where(inside, (c[:, 2] * ext[1] + c[:, 1]) * ext[0] + c[:, 0], -1)
    idx = np.nonzero(inside)[0]
    uk, first = np.unique(key[idx], return_index=True)
    first = idx[first]
    order = np.argsort(first, kind="stable")                 # voxels by first appearance
    uk, first = uk[order][:max_voxels], first[order][:max_voxels]
    vid_of = {int(k): v for v, k in enumerate(uk)}
    vid = np.array([vid_of.get(int(k), -1) if k >= 0 else -1 for k in key])
    srt = np.argsort(np.where(vid >= 0, vid, len(uk)), kind="stable")
    rank = np.zeros(len(pts), np.int64)
    seg = vid[srt]
    for j in range(1, len(srt)):
        if seg[j] == seg[j - 1]:
            rank[srt[j]] = rank[srt[j - 1]] + 1
    pcid = np.where((vid >= 0) & (rank < max_points), vid, -1)
    Vn = len(uk)
    vox = np.zeros((Vn, max_points, pts.shape[1]), np.float32)
    num = np.bincount(pcid[pcid >= 0], minlength=Vn).astype(np.int32)
    kept = np.nonzero(pcid >= 0)[0]
    vox[pcid[kept], rank[kept]] = pts[kept]
    if empty_mean:
        for v in range(Vn):
            vox[v, num[v]:] = (vox[v, :num[v]].astype(np.float64).sum(0) / num[v]).astype(np.float32)
    coords = c[first][:, ::-1].astype(np.int32)
    return vox, coords, num, pcid.astype(np.int32)


@pytest.mark.parametrize("seed,n,max_voxels,max_points,empty_mean", [
    (210, 3000, 10000, 4, True), (211, 3000, 50, 3, False), (212, 500, 1000, 40, True),
])
def test_vectorised_formulation_agrees(seed, n, max_voxels, max_points, empty_mean):
    r = W.rng(seed)
    pts = np.concatenate([r.uniform(-1.2, 1.2, (n, 3)), r.standard_normal((n, 1))], 1).astype(np.float32)
    args = ([0.25, 0.25, 0.5], [-1, -1, -1, 1, 1, 1], max_voxels, max_points, empty_mean)
    got = V.point_to_voxel(pts, *args)
    want = _vectorised(pts, *args)
    for g, w in zip(got, want):
        np.testing.assert_array_equal(g, w)


def test_page_example_invariants():
    pts = W.rng(220).uniform(-10, 10, (1000, 3)).astype(np.float32)
    vox, coords, num, pcid = V.point_to_voxel(pts, PAGE["vsize_xyz"], PAGE["range_xyz"], 5000, 5)
    c, inside = V.voxel_coords(pts, PAGE["vsize_xyz"], PAGE["range_xyz"])
    assert len({tuple(x) for x in coords}) == len(coords)                 # distinct voxels
    assert ((num >= 1) & (num <= 5)).all() and num.sum() == (pcid >= 0).sum()
    assert ((pcid >= 0) == inside).all()                                   # room for every inside point here
    np.testing.assert_array_equal(coords[pcid[inside]], c[inside][:, ::-1])  # each point in its own voxel (ZYX)
    firsts = [np.nonzero(pcid == v)[0][0] for v in range(len(coords))]
    assert (np.diff(firsts) > 0).all()                                     # ids by first appearance
    v = int(np.argmax(num < 5))
    np.testing.assert_allclose(vox[v, num[v]:], np.repeat(pts[pcid == v].mean(0, keepdims=True), 5 - num[v], 0),
                               rtol=1e-6)


def test_gather_by_voxel_id():
    f = np.arange(12, dtype=np.float32).reshape(4, 3)
    np.testing.assert_array_equal(V.gather_by_voxel_id(f, [2, -1, 0, 2]), [[6, 7, 8], [0, 0, 0], [0, 1, 2], [6, 7, 8]])
