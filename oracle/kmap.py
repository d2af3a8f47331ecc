"""Oracle kernel maps (test infrastructure only; see the package docstring).

Geometry shared by both kinds of convolution.  Output site ``o`` (per spatial
axis) reads the input at ``o * stride - pad + k * dil`` for kernel index
``k`` in ``[0, ksize)`` (torch ``conv3d`` cross-correlation; spconv USAGE.md,
"Core Concepts": a sparse convolution equals the dense convolution of the
densified tensor).  The flat offset index is ``(kz * ky_n + ky) * kx_n + kx``,
z slowest, which is the C order over (dz, dy, dx) of the MLX ``sparse/conv.py``
page's ``_kernel_offsets``.  A submanifold convolution is the case
``stride = 1, pad = ksize // 2, dil = 1`` whose output sites are the input
sites (spconv USAGE.md, "Submanifold Convolution"), so its offset ``d = k - ksize//2``
reads the input at ``c + d`` (MLX page, module docstring formula).

Readings taken where the pages are silent:
* a neighbour outside the spatial shape is absent (it cannot be occupied);
* the batch index never shifts, so no pair crosses samples (MLX page,
  ``build_indice_map``: the batch column is not offset);
* strided output rows are ordered by ascending (b, z, y, x);
* an output site outside ``[0, out_shape)`` is dropped, so the output may be
  empty (spconv COMMON_PROBLEMS.md, the ``[8, 200, 200]`` example).
"""

from __future__ import annotations

import numpy as np

MISSING = -1


def _triple(v) -> tuple:
    if np.isscalar(v):
        return (int(v),) * 3
    t = tuple(int(a) for a in v)
    assert len(t) == 3
    return t


def kernel_index_grid(ksize) -> np.ndarray:
    """``[K, 3]`` kernel indices (kz, ky, kx), z slowest (MLX page, ``_kernel_offsets``)."""
    kz, ky, kx = _triple(ksize)
    g = np.meshgrid(np.arange(kz), np.arange(ky), np.arange(kx), indexing="ij")
    return np.stack(g, axis=-1).reshape(-1, 3).astype(np.int64)


def subm_offsets(ksize) -> np.ndarray:
    """Centred offsets ``d = k - ksize // 2`` in the same order (MLX page, ``_kernel_offsets``)."""
    return kernel_index_grid(ksize) - np.array([s // 2 for s in _triple(ksize)])


def out_shape(shape, ksize, stride, pad, dil) -> tuple:
    """Per-axis output extent ``floor((S + 2p - dil (k - 1) - 1) / s) + 1`` (torch conv3d rule)."""
    out = []
    for S, k, s, p, d in zip(_triple(shape), _triple(ksize), _triple(stride), _triple(pad), _triple(dil)):
        out.append((S + 2 * p - d * (k - 1) - 1) // s + 1)
    return tuple(out)


def pack(coords: np.ndarray, shape) -> np.ndarray:
    """One int64 key per (b, z, y, x): ``((b Z + z) Y + y) X + x`` (MLX page, ``encode``)."""
    Z, Y, X = _triple(shape)
    c = coords.astype(np.int64)
    return ((c[:, 0] * Z + c[:, 1]) * Y + c[:, 2]) * X + c[:, 3]


def in_bounds(zyx: np.ndarray, shape) -> np.ndarray:
    return np.all((zyx >= 0) & (zyx < np.array(_triple(shape))), axis=1)


def coord_errors(coords: np.ndarray, batch: int, shape) -> dict:
    """Duplicate and out-of-range rows (undefined on the pages; the library rejects them)."""
    c = np.asarray(coords, dtype=np.int64).reshape(-1, 4)
    bad = ~(in_bounds(c[:, 1:], shape) & (c[:, 0] >= 0) & (c[:, 0] < batch))
    keys = pack(c[~bad], shape)
    dup = np.unique(keys).size != keys.size
    return {"out_of_range": bool(bad.any()), "duplicate": bool(dup)}


class SortedKeys:
    """Sorted packed keys with binary search: the lookup of the MLX page's
    ``build_indice_map`` (stable argsort, then ``searchsorted`` and a hit test)."""

    def __init__(self, keys: np.ndarray):
        self.order = np.argsort(keys, kind="stable")
        self.sorted = keys[self.order]

    def lookup(self, q: np.ndarray) -> np.ndarray:
        n = self.sorted.size
        if n == 0:
            return np.full(q.shape, MISSING, dtype=np.int64)
        pos = np.clip(np.searchsorted(self.sorted, q), 0, n - 1)
        hit = self.sorted[pos] == q
        return np.where(hit, self.order[pos], MISSING)


def subm_kmap(coords: np.ndarray, shape, ksize) -> np.ndarray:
    """Submanifold neighbour map ``nbr[K, N]``: ``nbr[k][i] = j`` iff input row j sits
    at ``coords[i] + d_k`` in the same sample, else -1.

    Follows the MLX page's ``build_indice_map``: encode the keys, sort, and for
    each offset shift the spatial columns (never the batch), encode, binary-search
    and test for a hit.  Probes that leave the grid are misses.
    """
    c = np.asarray(coords, dtype=np.int64).reshape(-1, 4)
    offs = subm_offsets(ksize)
    n = c.shape[0]
    nbr = np.full((offs.shape[0], n), MISSING, dtype=np.int32)
    if n == 0:
        return nbr
    table = SortedKeys(pack(c, shape))
    for k, d in enumerate(offs):
        probe = c.copy()
        probe[:, 1:] += d
        ok = in_bounds(probe[:, 1:], shape)
        rows = np.full(n, MISSING, dtype=np.int64)
        rows[ok] = table.lookup(pack(probe[ok], shape))
        nbr[k] = rows
    return nbr


def strided_kmap(coords: np.ndarray, batch: int, shape, ksize, stride, pad, dil) -> dict:
    """Strided kernel map, written from the definition.

    * ``out_coords[M, 4]``: the sorted set of (b, o) such that some input row i
      and kernel index k satisfy ``o * s - p + k * dil = coords_zyx[i]`` on every
      axis with ``0 <= o < out_shape`` (spconv USAGE.md, "Sparse Convolution":
      output sites are those a dense convolution would compute from valid data).
    * ``nbr_out[K, M]``: the input row at ``o * s - p + k * dil``, else -1.
    * ``nbr_in[K, N]``: the output row that input i feeds through offset k, else -1.
    """
    c = np.asarray(coords, dtype=np.int64).reshape(-1, 4)
    oshape = out_shape(shape, ksize, stride, pad, dil)
    kidx = kernel_index_grid(ksize)
    s = np.array(_triple(stride))
    p = np.array(_triple(pad))
    dl = np.array(_triple(dil))
    K, n = kidx.shape[0], c.shape[0]

    # candidate outputs of every (input, offset): o = (c + p - k dil) / s, exact and in range
    cand_rows = []
    cand_valid = []
    for k in range(K):
        num = c[:, 1:] + p - kidx[k] * dl
        o = num // s
        valid = np.all(num % s == 0, axis=1) & in_bounds(o, oshape) if min(oshape) > 0 else np.zeros(n, bool)
        cand_rows.append(np.concatenate([c[:, :1], o], axis=1))
        cand_valid.append(valid)
    allc = np.concatenate([r[v] for r, v in zip(cand_rows, cand_valid)], axis=0).reshape(-1, 4)
    out_keys = np.unique(pack(allc, oshape)) if allc.shape[0] else np.zeros(0, np.int64)
    M = out_keys.size
    Z, Y, X = oshape
    out_coords = np.stack([out_keys // (Z * Y * X), (out_keys // (Y * X)) % Z,
                           (out_keys // X) % Y, out_keys % X], axis=1).astype(np.int32).reshape(-1, 4)

    in_table = SortedKeys(pack(c, shape))
    oc = out_coords.astype(np.int64)
    nbr_out = np.full((K, M), MISSING, dtype=np.int32)
    for k in range(K):
        src = oc[:, 1:] * s - p + kidx[k] * dl
        ok = in_bounds(src, shape)
        rows = np.full(M, MISSING, dtype=np.int64)
        q = np.concatenate([oc[ok, :1], src[ok]], axis=1)
        rows[ok] = in_table.lookup(pack(q, shape))
        nbr_out[k] = rows

    out_table = SortedKeys(out_keys)
    nbr_in = np.full((K, n), MISSING, dtype=np.int32)
    for k in range(K):
        v = cand_valid[k]
        rows = np.full(n, MISSING, dtype=np.int64)
        rows[v] = out_table.lookup(pack(cand_rows[k][v], oshape))
        nbr_in[k] = rows
    return {"out_coords": out_coords, "out_shape": oshape, "nbr_out": nbr_out, "nbr_in": nbr_in}


def pairs_from_map(nbr: np.ndarray):
    """CSR pair lists of an output-stationary map: for each offset k, the pairs
    ``(nbr[k][o], o)`` with ``nbr[k][o] >= 0`` in ascending o.

    Returns ``pair_ptr[K + 1]`` (offset k owns ``[pair_ptr[k], pair_ptr[k+1])``),
    ``pair_in`` and ``pair_out``, all int32.
    """
    K = nbr.shape[0]
    ptr = np.zeros(K + 1, dtype=np.int64)
    ins, outs = [], []
    for k in range(K):
        o = np.nonzero(nbr[k] >= 0)[0]
        ins.append(nbr[k][o])
        outs.append(o)
        ptr[k + 1] = ptr[k] + o.size
    cat = (lambda xs: np.concatenate(xs).astype(np.int32)) if K else (lambda xs: np.zeros(0, np.int32))
    return ptr.astype(np.int32), cat(ins), cat(outs)
