"""GPU point-cloud voxelisation vs the oracle: voxel coordinates, counts,
point ids and stored points bit for bit (integer decisions on the same fp32
arithmetic, copies of the points), the empty-mean padding within fp32
rounding; and the gather of voxel features back to the points."""

import numpy as np
import pytest
import torch

import sparse_convolution_hash_amd as spc
import workloads as W
from oracle import voxel as V
from tests.parity import cuda, host

pytestmark = pytest.mark.gpu


def check(pts, vsize, rng_xyz, max_voxels, max_points, empty_mean, what=""):
    print(f"point_to_voxel {what} n={pts.shape[0]} F={pts.shape[1]} max_voxels={max_voxels} "
          f"max_points={max_points} mean={empty_mean}", flush=True)
    vox, coords, num, pcid = spc.point_to_voxel(cuda(pts), vsize, rng_xyz, max_voxels, max_points, empty_mean,
                                                with_id=True)
    rv, rc, rn, rp = V.point_to_voxel(pts, vsize, rng_xyz, max_voxels, max_points, empty_mean)
    assert vox.shape[0] == rv.shape[0]
    assert np.array_equal(host(coords), rc)
    assert np.array_equal(host(num), rn)
    assert np.array_equal(host(pcid), rp)
    gv = host(vox)
    stored = np.arange(max_points)[None, :] < rn[:, None]
    assert np.array_equal(gv[stored], rv[stored])
    np.testing.assert_allclose(gv[~stored], rv[~stored], rtol=2e-6, atol=1e-6)
    again = spc.point_to_voxel(cuda(pts), vsize, rng_xyz, max_voxels, max_points, empty_mean, with_id=True)
    assert all(torch.equal(a, b) for a, b in zip(again, (vox, coords, num, pcid)))  # run-to-run identical
    return vox, coords, num, pcid


@pytest.mark.parametrize("seed,n,F,max_voxels,max_points,empty_mean", [
    (230, 3000, 4, 10000, 4, True), (231, 3000, 3, 50, 3, False), (232, 500, 5, 1000, 40, True),
    (233, 20000, 4, 600, 2, True),
])
def test_random_clouds(seed, n, F, max_voxels, max_points, empty_mean):
    r = W.rng(seed)
    pts = np.concatenate([r.uniform(-1.2, 1.2, (n, 3)), r.standard_normal((n, F - 3))], 1).astype(np.float32)
    check(pts, [0.25, 0.25, 0.5], [-1, -1, -1, 1, 1, 1], max_voxels, max_points, empty_mean)


def test_page_example_configuration():
    pts = W.rng(234).uniform(-10, 10, (1000, 3)).astype(np.float32)
    check(pts, [0.1, 0.1, 0.1], [-80, -80, -2, 80, 80, 6], 5000, 5, True, "page example")


def test_boundaries_nan_and_empty():
    # points exactly on the box faces and voxel faces, and a NaN
    pts = np.array([[0, 0, 0], [1, 1, 1], [0.999999, 0, 0], [-1e-7, 0, 0], [0.5, 0.5, 0.5], [np.nan, 0, 0],
                    [0.25, 0.25, 0.25], [0.75, 0.5, 0.25]], np.float32)
    check(pts, [0.25, 0.25, 0.25], [0, 0, 0, 1, 1, 1], 100, 3, True, "faces")
    vox, coords, num = spc.point_to_voxel(torch.empty((0, 4), device="cuda"), [1, 1, 1], [0, 0, 0, 2, 2, 2], 10, 2)
    assert vox.shape == (0, 2, 4) and coords.shape == (0, 3) and num.shape == (0,)
    with pytest.raises(spc.SpcError):
        spc.point_to_voxel(torch.zeros((4, 2), device="cuda"), [1, 1, 1], [0, 0, 0, 2, 2, 2], 10, 2)
    with pytest.raises(spc.SpcError):
        spc.point_to_voxel(torch.zeros((4, 3), device="cuda"), [0, 1, 1], [0, 0, 0, 2, 2, 2], 10, 2)


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
def test_gather_by_voxel_id(dtype):
    r = W.rng(235)
    pts = np.concatenate([r.uniform(-1.2, 1.2, (4000, 3)), r.uniform(0, 1, (4000, 1))], 1).astype(np.float32)
    _, _, _, pcid = spc.point_to_voxel(cuda(pts), [0.25, 0.25, 0.5], [-1, -1, -1, 1, 1, 1], 100, 3, with_id=True)
    seg = torch.from_numpy(r.standard_normal((100, 48)).astype(np.float32)).to(dtype)
    got = spc.gather_by_voxel_id(cuda(seg), pcid)
    assert torch.equal(got.cpu(), torch.from_numpy(V.gather_by_voxel_id(seg.float().numpy(), host(pcid))).to(dtype))


def test_lidar_sweep():
    pts = W.lidar_points(W.rng(236))
    cfg = W.LIDAR_VOXEL
    vox, coords, num, pcid = check(pts, cfg["vsize_xyz"], cfg["range_xyz"], cfg["max_voxels"], cfg["max_points"],
                                   True, "lidar sweep")
    print(f"voxels {vox.shape[0]}, points kept {int((pcid >= 0).sum())} of {pts.shape[0]}", flush=True)
