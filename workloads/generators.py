"""Seeded synthetic voxel sets and tensors for sparse 3-D convolution.

Every generator draws from numpy ``Generator(PCG64)`` streams split off one
``SeedSequence(seed)`` (coordinates, features, weights, bias, gradient and a
second layer's weights each get their own stream), so a workload is a pure
function of its seed.  Coordinates are built as a set of unique sites and then
emitted in a seeded random row order: nothing downstream may assume the rows
are sorted.  Half-precision tensors are sampled in fp32 and cast with
round-to-nearest-even (torch's ``.to(dtype)``).

Coordinates are int32 ``[N, 4]`` rows ``(b, z, y, x)``, the batch index first,
as in spconv's ``SparseConvTensor`` (spconv USAGE.md, "Creating and Converting
SparseConvTensor").  Weights are ``[K^3, Cin, Cout]`` (the MLX
``sparse/conv.py`` page, ``SubMConv3d`` docstring).

The named workloads stand in for data the pages measure on but do not ship:
a LiDAR detection scene (spconv's 120k-voxel ``bench_basic`` size and the
BEVFusion SparseEncoder on the muSPACE operator matrix), mesh surfaces on a
128^3 grid (the MLX page's 128^3 / 128-channel run) and a sparse U-Net training
step (the MinkowskiEngine performance guide).  No dataset item is reproduced.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

_STREAMS = ("coords", "feats", "weight", "bias", "grad", "weight2")


def _rngs(seed: int) -> dict:
    children = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {name: np.random.Generator(np.random.PCG64(s)) for name, s in zip(_STREAMS, children)}


def _to_dtype(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """fp32 numpy array -> torch CPU tensor of ``dtype`` (RNE for fp16/bf16)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dtype)


# --------------------------------------------------------------------------
# coordinate sets
# --------------------------------------------------------------------------

def _shuffle_rows(rng: np.random.Generator, coords: np.ndarray) -> np.ndarray:
    perm = rng.permutation(coords.shape[0])
    return np.ascontiguousarray(coords[perm], dtype=np.int32)


def uniform_grid(rng: np.random.Generator, n: int, side: int, batch: int = 1) -> np.ndarray:
    """``n`` unique sites per sample drawn uniformly without replacement from side^3."""
    rows = []
    for b in range(batch):
        lin = rng.choice(side ** 3, size=n, replace=False)
        z, y, x = np.unravel_index(lin, (side, side, side))
        rows.append(np.stack([np.full(n, b), z, y, x], axis=1))
    return _shuffle_rows(rng, np.concatenate(rows, axis=0))


def lidar_scene(rng: np.random.Generator, batch: int = 2, shape=(41, 1600, 1408),
                per_sample: int = 60000, ground_frac: float = 0.7, blobs: int = 100,
                sigma: float = 3.0) -> np.ndarray:
    """Ground plane plus Gaussian blobs, the shape of a LiDAR voxel grid.

    Per sample: ``ground_frac * per_sample`` unique sites on the two z-planes
    {2, 3} with (y, x) uniform; the rest split evenly over ``blobs`` blobs whose
    centres are uniform in the grid.  A blob draws ``round(N(centre, sigma^2))``
    per axis, clipped to the grid, and keeps a draw only if the site is not yet
    taken, until it holds its share.
    """
    Z, Y, X = shape
    n_ground = int(round(per_sample * ground_frac))
    n_blob_total = per_sample - n_ground
    per_blob = n_blob_total // blobs
    extra = n_blob_total - per_blob * blobs
    hi = np.array([Z - 1, Y - 1, X - 1])
    rows = []
    for b in range(batch):
        lin = rng.choice(2 * Y * X, size=n_ground, replace=False)
        gz = 2 + lin // (Y * X)
        rem = lin % (Y * X)
        gy, gx = rem // X, rem % X
        ground = np.stack([gz, gy, gx], axis=1)
        taken = set(((ground[:, 0] * Y + ground[:, 1]) * X + ground[:, 2]).tolist())
        centres = rng.uniform(0.0, 1.0, size=(blobs, 3)) * np.array([Z, Y, X])
        blob_pts = []
        for j in range(blobs):
            want = per_blob + (1 if j < extra else 0)
            got = 0
            while got < want:
                draw = np.rint(centres[j] + sigma * rng.standard_normal((256, 3))).astype(np.int64)
                draw = np.clip(draw, 0, hi)
                for p in draw:
                    key = (int(p[0]) * Y + int(p[1])) * X + int(p[2])
                    if key in taken:
                        continue
                    taken.add(key)
                    blob_pts.append(p)
                    got += 1
                    if got == want:
                        break
        pts = np.concatenate([ground, np.asarray(blob_pts, dtype=np.int64).reshape(-1, 3)], axis=0)
        rows.append(np.concatenate([np.full((pts.shape[0], 1), b), pts], axis=1))
    return _shuffle_rows(rng, np.concatenate(rows, axis=0))


def mesh_shells(rng: np.random.Generator, batch: int = 4, side: int = 128, shells: int = 8,
                rmin: float = 10.0, rmax: float = 50.0) -> np.ndarray:
    """Union of ``shells`` one-voxel-thick sphere shells per sample on a side^3 grid.

    A shell has radius r ~ U[rmin, rmax] and a centre uniform in [0, side)^3;
    the integer site v belongs to it iff r - 1/2 <= |v - centre| < r + 1/2.
    Sites outside the grid are clipped away; shells of one sample are united.
    """
    rows = []
    for b in range(batch):
        keys = []
        for _ in range(shells):
            r = rng.uniform(rmin, rmax)
            c = rng.uniform(0.0, float(side), size=3)
            lo = np.maximum(0, np.floor(c - r - 1.0)).astype(np.int64)
            hi = np.minimum(side - 1, np.ceil(c + r + 1.0)).astype(np.int64)
            zz = np.arange(lo[0], hi[0] + 1)
            yy = np.arange(lo[1], hi[1] + 1)
            xx = np.arange(lo[2], hi[2] + 1)
            dz2 = (zz - c[0])[:, None, None] ** 2
            dy2 = (yy - c[1])[None, :, None] ** 2
            dx2 = (xx - c[2])[None, None, :] ** 2
            d = np.sqrt(dz2 + dy2 + dx2)
            z, y, x = np.nonzero((d >= r - 0.5) & (d < r + 0.5))
            keys.append(((zz[z] * side + yy[y]) * side + xx[x]).astype(np.int64))
        u = np.unique(np.concatenate(keys))
        z, y, x = np.unravel_index(u, (side, side, side))
        rows.append(np.stack([np.full(u.shape[0], b), z, y, x], axis=1))
    return _shuffle_rows(rng, np.concatenate(rows, axis=0))


# Point-cloud voxelisation on a LiDAR-like sweep: 0.1 x 0.1 x 0.2 m voxels
# over +-51.2 m (x, y) and [-5, 3) m (z), at most 10 points per voxel and
# 160k voxels (a common detection-network setting; no dataset is read).
LIDAR_VOXEL = dict(vsize_xyz=[0.1, 0.1, 0.2], range_xyz=[-51.2, -51.2, -5.0, 51.2, 51.2, 3.0],
                   max_voxels=160_000, max_points=10)


def lidar_points(rng: np.random.Generator, n: int = 200_000, features: int = 4) -> np.ndarray:
    """A synthetic sweep ``[n, features]`` fp32 (x, y, z, intensity, ...): 65%
    ground returns around the sensor (range uniform in [1, 60] m, so the
    density falls as 1/range and the far ones leave the box; azimuth uniform;
    z = -1.7 m with 3 cm noise), 35% object returns in 150 Gaussian blobs
    (centres uniform over +-45 m, z in [-1.5, 0.5] m, spread 0.6 / 0.6 / 0.4 m);
    further features uniform in [0, 1); rows in a seeded random order."""
    ng = int(n * 0.65)
    no = n - ng
    rad, az = rng.uniform(1, 60, ng), rng.uniform(0, 2 * np.pi, ng)
    ground = np.stack([rad * np.cos(az), rad * np.sin(az), -1.7 + 0.03 * rng.standard_normal(ng)], 1)
    centres = np.stack([rng.uniform(-45, 45, 150), rng.uniform(-45, 45, 150), rng.uniform(-1.5, 0.5, 150)], 1)
    which = rng.integers(0, 150, no)
    objects = centres[which] + rng.standard_normal((no, 3)) * np.array([0.6, 0.6, 0.4])
    xyz = np.concatenate([ground, objects])[rng.permutation(n)]
    extra = rng.uniform(0, 1, (n, features - 3))
    return np.concatenate([xyz, extra], 1).astype(np.float32)


def tiny_grid(rng: np.random.Generator, side: int, fill: float, batch: int = 1) -> np.ndarray:
    """Each site of a side^3 grid per sample kept independently with probability ``fill``."""
    rows = []
    for b in range(batch):
        keep = rng.random(side ** 3) < fill
        z, y, x = np.unravel_index(np.nonzero(keep)[0], (side, side, side))
        rows.append(np.stack([np.full(z.shape[0], b), z, y, x], axis=1))
    return _shuffle_rows(rng, np.concatenate(rows, axis=0).reshape(-1, 4))


def random_block(rng: np.random.Generator, n: int, origin=(0, 0, 0), b: int = 0) -> np.ndarray:
    """All n^3 sites of a full block at ``origin``, rows in a seeded random order."""
    z, y, x = np.meshgrid(*(np.arange(n) + o for o, n in zip(origin, (n, n, n))), indexing="ij")
    c = np.stack([np.full(z.size, b), z.ravel(), y.ravel(), x.ravel()], axis=1)
    return _shuffle_rows(rng, c)


# --------------------------------------------------------------------------
# named workloads
# --------------------------------------------------------------------------

@dataclass
class Workload:
    """One layer's inputs: coordinates, geometry and tensors (torch CPU)."""

    name: str
    coords: np.ndarray               # int32 [N, 4] (b, z, y, x)
    batch: int
    shape: tuple                     # spatial shape (Z, Y, X)
    ksize: int
    stride: int
    pad: int
    dil: int
    subm: bool
    cin: int
    cout: int
    dtype: torch.dtype
    feats: torch.Tensor              # [N, cin] dtype
    weight: torch.Tensor             # [K, cin, cout] dtype
    bias: Optional[torch.Tensor] = None    # [cout] fp32
    grad: Optional[torch.Tensor] = None    # [n_out, cout] dtype (drawn when the output size is known)
    extra: dict = field(default_factory=dict)

    @property
    def n(self) -> int:
        return int(self.coords.shape[0])

    @property
    def K(self) -> int:
        return self.ksize ** 3


WORKLOAD_NAMES = (
    "subm_k3_f32_uniform32",       # 2,000 sites of 32^3, 16 -> 16 fp32, bias
    "subm_k3_f16_lidar120k",       # 2 x 60k LiDAR-like sites on 41x1600x1408, 64 -> 64 fp16
    "subm_k3_k1_bf16_shells128",   # 4 samples of mesh shells on 128^3, 128 -> 128 bf16, then k=1
    "strided_k3s2_f16_lidar120k",  # k3 s2 p1 on the LiDAR sites, 64 -> 128 fp16
    "train_subm_k3_bf16_shells96", # fwd + dinput + dfilter on the shell sites, 96 -> 96 bf16
)


def _normal(rng, shape, std=1.0):
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def workload(name: str, with_grad: bool = False) -> Workload:
    """Build a named workload.  Seeds are fixed per workload (1..5 in the order above)."""
    if name == "subm_k3_f32_uniform32":
        g = _rngs(1)
        coords = uniform_grid(g["coords"], 2000, 32)
        n, cin, cout = coords.shape[0], 16, 16
        w = workload_tensors(g, n, cin, cout, 27, torch.float32, std=1.0 / np.sqrt(27 * cin),
                             bias_std=0.1, with_grad=with_grad)
        return Workload(name, coords, 1, (32, 32, 32), 3, 1, 1, 1, True, cin, cout,
                        torch.float32, **w)
    if name in ("subm_k3_f16_lidar120k", "strided_k3s2_f16_lidar120k"):
        g = _rngs(2)
        coords = lidar_scene(g["coords"])
        n = coords.shape[0]
        feats = _to_dtype(_normal(g["feats"], (n, 64)), torch.float16)
        if name == "subm_k3_f16_lidar120k":
            w = _to_dtype(_normal(g["weight"], (27, 64, 64), 1.0 / np.sqrt(27 * 64)), torch.float16)
            grad = _to_dtype(_normal(g["grad"], (n, 64)), torch.float16) if with_grad else None
            wl = Workload(name, coords, 2, (41, 1600, 1408), 3, 1, 1, 1, True, 64, 64,
                          torch.float16, feats, w, None, grad)
            # a following k=1 layer (per-voxel linear, 64 -> 64)
            wl.extra["weight_k1"] = _to_dtype(_normal(g["weight2"], (1, 64, 64), 1.0 / np.sqrt(64)),
                                              torch.float16)
            return wl
        g4 = _rngs(4)
        w = _to_dtype(_normal(g4["weight"], (27, 64, 128), 1.0 / np.sqrt(27 * 64)), torch.float16)
        wl = Workload(name, coords, 2, (41, 1600, 1408), 3, 2, 1, 1, False, 64, 128,
                      torch.float16, feats, w)
        wl.extra["grad_rng"] = g4["grad"]
        return wl
    if name == "subm_k3_k1_bf16_shells128":
        g = _rngs(3)
        coords = mesh_shells(g["coords"])
        n = coords.shape[0]
        feats = _to_dtype(_normal(g["feats"], (n, 128)), torch.bfloat16)
        w = _to_dtype(_normal(g["weight"], (27, 128, 128), 1.0 / np.sqrt(27 * 128)), torch.bfloat16)
        w1 = _to_dtype(_normal(g["weight2"], (1, 128, 128), 1.0 / np.sqrt(128)), torch.bfloat16)
        wl = Workload(name, coords, 4, (128, 128, 128), 3, 1, 1, 1, True, 128, 128,
                      torch.bfloat16, feats, w)
        wl.extra["weight_k1"] = w1
        return wl
    if name == "train_subm_k3_bf16_shells96":
        coords = mesh_shells(_rngs(3)["coords"])
        g = _rngs(5)
        n = coords.shape[0]
        feats = _to_dtype(_normal(g["feats"], (n, 96)), torch.bfloat16)
        w = _to_dtype(_normal(g["weight"], (27, 96, 96), 1.0 / np.sqrt(27 * 96)), torch.bfloat16)
        grad = _to_dtype(_normal(g["grad"], (n, 96)), torch.bfloat16)
        return Workload(name, coords, 4, (128, 128, 128), 3, 1, 1, 1, True, 96, 96,
                        torch.bfloat16, feats, w, None, grad)
    raise KeyError(f"unknown workload {name!r}; known: {WORKLOAD_NAMES}")


def workload_tensors(g: dict, n: int, cin: int, cout: int, K: int, dtype: torch.dtype,
                     std: float, bias_std: Optional[float] = None, with_grad: bool = False) -> dict:
    """Features, weight, optional fp32 bias and optional gradient for an n-row layer."""
    out = {
        "feats": _to_dtype(_normal(g["feats"], (n, cin)), dtype),
        "weight": _to_dtype(_normal(g["weight"], (K, cin, cout), std), dtype),
        "bias": None,
        "grad": None,
    }
    if bias_std is not None:
        out["bias"] = torch.from_numpy(_normal(g["bias"], (cout,), bias_std))
    if with_grad:
        out["grad"] = _to_dtype(_normal(g["grad"], (n, cout)), dtype)
    return out


def small_layer(seed: int, coords: np.ndarray, cin: int, cout: int, K: int, dtype: torch.dtype,
                bias: bool = True, n_out: Optional[int] = None) -> dict:
    """Tensors for a small test layer on given coordinates (gradient sized ``n_out``)."""
    g = _rngs(seed)
    n = coords.shape[0]
    t = workload_tensors(g, n, cin, cout, K, dtype, std=1.0 / np.sqrt(K * cin),
                         bias_std=0.1 if bias else None)
    m = n if n_out is None else n_out
    t["grad"] = _to_dtype(_normal(g["grad"], (m, cout)), dtype)
    return t


def grad_for(rng: np.random.Generator, n_out: int, cout: int, dtype: torch.dtype) -> torch.Tensor:
    """Upstream gradient ~N(0, 1) for an output of ``n_out`` rows."""
    return _to_dtype(_normal(rng, (n_out, cout)), dtype)


def rng(seed: int, stream: str = "coords") -> np.random.Generator:
    """One named stream of ``seed`` (for tests that draw their own coordinates)."""
    return _rngs(seed)[stream]
