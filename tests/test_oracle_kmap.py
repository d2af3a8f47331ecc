"""Pins of the oracle's kernel maps against brute force, closed forms, the
spconv worked example, invariants and torch's dense conv3d (CPU only)."""

import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workloads as W
from oracle import kmap as O
from tests.dense import densify

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- brute force

def brute_subm(coords, shape, k):
    """O(N^2 K) enumeration: for every row and offset, scan all rows."""
    r = k // 2
    offs = [(a - r, b - r, c - r) for a in range(k) for b in range(k) for c in range(k)]
    n = len(coords)
    nbr = np.full((len(offs), n), -1, dtype=np.int32)
    for i in range(n):
        b, z, y, x = (int(v) for v in coords[i])
        for kk, (dz, dy, dx) in enumerate(offs):
            q = (b, z + dz, y + dy, x + dx)
            for j in range(n):
                if tuple(int(v) for v in coords[j]) == q:
                    nbr[kk, i] = j
    return nbr


def brute_strided(coords, batch, shape, k, s, p, d):
    """Enumerate every output site of the dense output grid in (b, z, y, x) order
    and every kernel index; keep sites that some input reaches."""
    osh = O.out_shape(shape, k, s, p, d)
    lut = {tuple(int(v) for v in c): i for i, c in enumerate(coords)}
    outs, rows = [], []
    for b in range(batch):
        for oz in range(max(osh[0], 0)):
            for oy in range(max(osh[1], 0)):
                for ox in range(max(osh[2], 0)):
                    col = []
                    for kz in range(k):
                        for ky in range(k):
                            for kx in range(k):
                                q = (b, oz * s - p + kz * d, oy * s - p + ky * d, ox * s - p + kx * d)
                                col.append(lut.get(q, -1))
                    if any(v >= 0 for v in col):
                        outs.append((b, oz, oy, ox))
                        rows.append(col)
    K = k ** 3
    nbr_out = np.array(rows, dtype=np.int32).T.reshape(K, len(outs))
    nbr_in = np.full((K, len(coords)), -1, dtype=np.int32)
    for o in range(len(outs)):
        for kk in range(K):
            if nbr_out[kk, o] >= 0:
                nbr_in[kk, nbr_out[kk, o]] = o
    return np.array(outs, dtype=np.int32).reshape(-1, 4), nbr_out, nbr_in


@pytest.mark.parametrize("seed,side,fill,batch,k", [
    (11, 5, 0.3, 1, 3), (12, 6, 0.05, 2, 3), (13, 4, 0.6, 3, 3), (14, 5, 0.25, 1, 5),
    (15, 7, 0.15, 2, 1), (16, 6, 0.4, 1, 3),
])
def test_subm_matches_brute_force(seed, side, fill, batch, k):
    c = W.tiny_grid(W.rng(seed), side, fill, batch)
    assert np.array_equal(O.subm_kmap(c, (side,) * 3, k), brute_subm(c, (side,) * 3, k))


@pytest.mark.parametrize("seed,shape,fill,batch,k,s,p,d", [
    (21, (6, 5, 7), 0.2, 1, 3, 2, 1, 1),
    (22, (7, 7, 7), 0.1, 2, 3, 2, 0, 1),
    (23, (8, 6, 5), 0.15, 1, 2, 2, 0, 1),
    (24, (6, 6, 6), 0.2, 1, 3, 1, 1, 2),
    (25, (9, 7, 8), 0.1, 2, 3, 3, 2, 1),
    (26, (5, 5, 5), 0.3, 1, 3, 1, 0, 1),
])
def test_strided_matches_brute_force(seed, shape, fill, batch, k, s, p, d):
    r = W.rng(seed)
    rows = []
    for b in range(batch):
        keep = r.random(int(np.prod(shape))) < fill
        z, y, x = np.unravel_index(np.nonzero(keep)[0], shape)
        rows.append(np.stack([np.full(z.size, b), z, y, x], 1))
    c = np.concatenate(rows).astype(np.int32)
    c = c[r.permutation(c.shape[0])]
    got = O.strided_kmap(c, batch, shape, k, s, p, d)
    oc, no, ni = brute_strided(c, batch, shape, k, s, p, d)
    assert np.array_equal(got["out_coords"], oc)
    assert np.array_equal(got["nbr_out"], no)
    assert np.array_equal(got["nbr_in"], ni)


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("n", [1, 2, 4, 5])
def test_full_block_hit_counts(n):
    c = W.random_block(W.rng(30 + n), n, origin=(2, 3, 1))
    nbr = O.subm_kmap(c, (10, 10, 10), 3)
    offs = O.subm_offsets(3)
    for k, d in enumerate(offs):
        assert (nbr[k] >= 0).sum() == np.prod([n - abs(int(a)) for a in d])
    assert (nbr >= 0).sum() == (3 * n - 2) ** 3          # n = 4 gives 1000


def test_single_voxel_centre_only():
    c = np.array([[0, 3, 3, 3]], dtype=np.int32)
    nbr = O.subm_kmap(c, (8, 8, 8), 3)
    assert (nbr >= 0).sum() == 1 and nbr[13, 0] == 0


def test_golden_empty_strided_output():
    g = json.load(open(os.path.join(GOLDEN, "empty_strided_output.json")))
    res = O.strided_kmap(np.array(g["coords"], np.int32), g["batch"], g["spatial_shape"],
                         g["ksize"], g["stride"], g["padding"], g["dilation"])
    assert res["out_coords"].shape[0] == g["expected_n_out"]
    assert res["nbr_out"].shape == (27, 0)
    assert (res["nbr_in"] == -1).all()


def test_strided_interior_pair_count():
    # k=3, s=2, p=1: along an axis an odd coordinate reaches 2 outputs, an even one 1
    shape = (41, 1600, 1408)
    for z, y, x in [(5, 100, 200), (6, 101, 200), (7, 99, 301), (8, 100, 202)]:
        res = O.strided_kmap(np.array([[0, z, y, x]], np.int32), 1, shape, 3, 2, 1, 1)
        want = np.prod([2 if v % 2 else 1 for v in (z, y, x)])
        assert (res["nbr_in"] >= 0).sum() == want == res["out_coords"].shape[0]
    # upper edge: y = 1599 would need o_y = 800 = out extent, so that output is dropped
    res = O.strided_kmap(np.array([[0, 6, 1599, 200]], np.int32), 1, shape, 3, 2, 1, 1)
    assert res["out_shape"] == (21, 800, 704)
    assert (res["nbr_in"] >= 0).sum() == 1


def test_out_shape_rule():
    assert O.out_shape((41, 1600, 1408), 3, 2, 1, 1) == (21, 800, 704)
    assert O.out_shape((8, 200, 200), 3, 2, (0, 1, 1), 1) == (3, 100, 100)
    assert O.out_shape((10, 10, 10), 3, 1, 0, 2) == (6, 6, 6)


# ---------------------------------------------------------------- invariants

def test_subm_symmetry_and_centre():
    c = W.tiny_grid(W.rng(40), 10, 0.3, 2)
    nbr = O.subm_kmap(c, (10, 10, 10), 3)
    K, n = nbr.shape
    assert np.array_equal(nbr[K // 2], np.arange(n))
    for k in range(K):
        hit = np.nonzero(nbr[k] >= 0)[0]
        assert np.array_equal(nbr[K - 1 - k][nbr[k][hit]], hit)


def test_strided_maps_are_transposes_and_pairs_are_nonzeros():
    c = W.tiny_grid(W.rng(41), 11, 0.2, 2)
    res = O.strided_kmap(c, 2, (11, 11, 11), 3, 2, 1, 1)
    no, ni = res["nbr_out"], res["nbr_in"]
    for k in range(no.shape[0]):
        o = np.nonzero(no[k] >= 0)[0]
        assert np.array_equal(ni[k][no[k][o]], o)
        assert (ni[k] >= 0).sum() == o.size
    ptr, pin, pout = O.pairs_from_map(no)
    assert ptr[-1] == (no >= 0).sum()
    for k in range(no.shape[0]):
        seg = slice(ptr[k], ptr[k + 1])
        assert np.all(np.diff(pout[seg]) > 0)
        assert np.array_equal(no[k][pout[seg]], pin[seg])
    # every output is reached by at least one input
    assert np.all((no >= 0).any(axis=0))


@pytest.mark.parametrize("k,s,p,d", [(3, 2, 1, 1), (2, 2, 0, 1), (3, 1, 0, 2), (3, 3, 1, 1)])
def test_strided_out_set_is_dense_support(k, s, p, d):
    shape = (9, 10, 8)
    c = W.tiny_grid(W.rng(50 + k + s), 8, 0.1, 2)
    res = O.strided_kmap(c, 2, shape, k, s, p, d)
    occ = densify(c, np.ones((c.shape[0], 1)), 2, shape)
    sup = F.conv3d(occ, torch.ones(1, 1, k, k, k, dtype=torch.float64), stride=s, padding=p, dilation=d)
    b, _, z, y, x = torch.nonzero(sup > 0.5, as_tuple=True)
    want = torch.stack([b, z, y, x], 1).numpy()
    assert res["out_shape"] == tuple(sup.shape[2:])
    assert np.array_equal(res["out_coords"], want)       # nonzero() is (b, z, y, x) order


def test_empty_input():
    c = np.zeros((0, 4), np.int32)
    assert O.subm_kmap(c, (4, 4, 4), 3).shape == (27, 0)
    res = O.strided_kmap(c, 1, (4, 4, 4), 3, 2, 1, 1)
    assert res["out_coords"].shape == (0, 4) and res["nbr_out"].shape == (27, 0)
    ptr, pin, pout = O.pairs_from_map(res["nbr_out"])
    assert ptr.tolist() == [0] * 28 and pin.size == 0


def test_coord_errors():
    shape = (4, 4, 4)
    assert O.coord_errors(np.array([[0, 1, 1, 1], [0, 1, 1, 2]]), 1, shape) == \
        {"out_of_range": False, "duplicate": False}
    assert O.coord_errors(np.array([[0, 1, 1, 1], [0, 1, 1, 1]]), 1, shape)["duplicate"]
    assert O.coord_errors(np.array([[0, 4, 1, 1]]), 1, shape)["out_of_range"]
    assert O.coord_errors(np.array([[1, 0, 0, 0]]), 1, shape)["out_of_range"]
    assert O.coord_errors(np.array([[0, 0, -1, 0]]), 1, shape)["out_of_range"]


def test_workload_kmaps_are_consistent():
    """Invariants hold at the full size of the small named workload."""
    w = W.workload("subm_k3_f32_uniform32")
    nbr = O.subm_kmap(w.coords, w.shape, 3)
    assert np.array_equal(nbr[13], np.arange(w.n))
    for k in range(27):
        hit = np.nonzero(nbr[k] >= 0)[0]
        assert np.array_equal(nbr[26 - k][nbr[k][hit]], hit)
