"""ctypes binding of libspc (include/spc.h): argument marshalling only.

Each function here has the name of the C entry point it wraps, takes torch
tensors that already live on the GPU, allocates the outputs and the workspace
with torch (device memory is all torch provides) and passes raw pointers and
the current HIP stream to the library.  Every step of the computation runs in
the library's HIP kernels; there is no CPU or PyTorch fallback, and a missing
``libspc.so`` raises.
"""

from __future__ import annotations

import ctypes
import functools
import os
from typing import Optional, Sequence

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspc.so")

SPC_OK, SPC_ERR_ARG, SPC_ERR_UNSUPPORTED, SPC_ERR_CAPACITY, SPC_ERR_COORD, SPC_ERR_WORKSPACE, SPC_ERR_HIP = range(7)
COORD_OUT_OF_RANGE, COORD_DUPLICATE = 1, 2
_DTYPES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
_STATUS = {1: "SPC_ERR_ARG", 2: "SPC_ERR_UNSUPPORTED", 3: "SPC_ERR_CAPACITY", 4: "SPC_ERR_COORD",
           5: "SPC_ERR_WORKSPACE", 6: "SPC_ERR_HIP"}

EXPORTS = ("spc_out_shape", "spc_kmap_workspace", "spc_build_kmap", "spc_build_kmap_async", "spc_subm_conv_fwd",
           "spc_sparse_conv_fwd", "spc_sparse_inverse_conv_fwd", "spc_conv_fwd_fused", "spc_transpose_weight",
           "spc_conv_fwd_wt", "spc_conv_fwd_dev_rows", "spc_conv_bwd_input",
           "spc_conv_bwd_filter_workspace",
           "spc_conv_bwd_filter", "spc_conv_bwd_filter_noalloc", "spc_sparse_maxpool_fwd", "spc_sparse_maxpool_bwd",
           "spc_point_to_voxel_workspace", "spc_point_to_voxel", "spc_gather_by_voxel_id", "spc_calibrate_mfma",
           "spc_last_error", "spc_version")


class SpcError(RuntimeError):
    def __init__(self, status: int, func: str, msg: str):
        super().__init__(f"{func}: {_STATUS.get(status, status)}: {msg}")
        self.status = status


class Geom(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("shape", ctypes.c_int32 * 3), ("ksize", ctypes.c_int32 * 3),
                ("stride", ctypes.c_int32 * 3), ("pad", ctypes.c_int32 * 3), ("dil", ctypes.c_int32 * 3),
                ("subm", ctypes.c_int32), ("table", ctypes.c_int32)]


TABLES = {"hash": 0, "grid": 1}   # SPC_TABLE_HASH, SPC_TABLE_GRID


def _t3(v) -> tuple:
    if isinstance(v, int):
        return (v, v, v)
    v = tuple(int(a) for a in v)
    if len(v) != 3:
        raise ValueError("expected an int or 3 ints")
    return v


def make_geom(batch: int, shape, ksize, stride=1, pad=0, dil=1, subm: bool = True, table: str = "hash") -> Geom:
    a = lambda v: (ctypes.c_int32 * 3)(*_t3(v))
    if table not in TABLES:
        raise ValueError(f"table must be one of {tuple(TABLES)}, got {table!r}")
    return Geom(int(batch), a(shape), a(ksize), a(stride), a(pad), a(dil), 1 if subm else 0, TABLES[table])


_lib = None
_P, _I64, _I32, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """The loaded libspc.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m sparse_convolution_hash_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    GP = ctypes.POINTER(Geom)
    sig = {
        "spc_out_shape": [GP, ctypes.POINTER(_I32)],
        "spc_kmap_workspace": [GP, _I64, ctypes.POINTER(_SZ)],
        "spc_build_kmap": [GP, _P, _I64, _P, _I64, ctypes.POINTER(_I64), _P, _P, _P, _P, _P, _I64, _P, _P, _P, _P,
                           _SZ, _P],
        "spc_build_kmap_async": [GP, _P, _I64, _P, _I64, _P, _P, _P, _P, _P, _P, _I64, _P, _P, _P, _P, _SZ, _P],
        "spc_subm_conv_fwd": [_I32, _P, _I64, _I32, _P, _I32, _I32, _P, _P, _P, _P, _P],
        "spc_sparse_conv_fwd": [_I32, _P, _I64, _I32, _P, _I32, _I32, _P, _P, _P, _I64, _P, _P],
        "spc_sparse_inverse_conv_fwd": [_I32, _P, _I64, _I32, _P, _I32, _I32, _P, _P, _P, _I64, _P, _P],
        "spc_conv_fwd_fused": [_I32, _P, _I64, _I32, _P, _I32, _I32, _P, _P, _P, _I64, _P, _I32, _P, _P],
        "spc_transpose_weight": [_I32, _P, _I32, _I32, _I32, _P, _P],
        "spc_conv_fwd_wt": [_I32, _P, _I64, _I32, _P, _I32, _I32, _P, _P, _I32, _P, _I64, _P, _I32, _P, _P],
        "spc_conv_fwd_dev_rows": [_I32, _P, _I64, _I32, _P, _I32, _I32, _I32, _P, _P, _P, _I64, _P, _P, _I32, _P,
                                  _P],
        "spc_conv_bwd_input": [_I32, _P, _I64, _I32, _P, _I32, _I32, _P, _I32, _P, _I64, _P, _P],
        "spc_conv_bwd_filter_workspace": [_I64, _I64, _I32, _I32, _I32, _I32, ctypes.POINTER(_SZ)],
        "spc_conv_bwd_filter": [_I32, _P, _I64, _I32, _P, _I64, _I32, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P],
        "spc_conv_bwd_filter_noalloc": [_I32, _P, _I64, _I32, _P, _I64, _I32, _I32, _P, _P, _P, _P, _P, _P],
        "spc_sparse_maxpool_fwd": [_I32, _P, _I64, _I32, _P, _I32, _I64, _P, _P, _P],
        "spc_sparse_maxpool_bwd": [_I32, _P, _I64, _I32, _P, _P, _I32, _I64, _P, _P],
        "spc_point_to_voxel_workspace": [_I64, _I32, _I64, _I32, ctypes.POINTER(_SZ)],
        "spc_point_to_voxel": [_P, _I64, _I32, _P, _P, _I64, _I32, _I32, _P, _P, _P, _P,
                               ctypes.POINTER(ctypes.c_int64), _P, _SZ, _P],
        "spc_gather_by_voxel_id": [_I32, _P, _I64, _I32, _P, _I64, _P, _P],
        "spc_calibrate_mfma": [_I32, _I32, _I32, _P, ctypes.POINTER(ctypes.c_double), _P],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    for name in ("spc_last_error", "spc_version"):
        f = getattr(L, name)
        f.argtypes = []
        f.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int, func: str):
    if status != SPC_OK:
        raise SpcError(status, func, lib().spc_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(dev: torch.device):
    """The current stream's handle on `dev` (torch's raw accessor when it has
    one: a Stream object per call costs host time on every launch)."""
    if _raw_stream is not None:
        return _raw_stream(dev.index if dev.index is not None else torch.cuda.current_device())
    return torch.cuda.current_stream(dev).cuda_stream


def _need(t: torch.Tensor, name: str, dtype=None, dev=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")


def version() -> str:
    return lib().spc_version().decode()


def out_shape(batch, shape, ksize, stride=1, pad=0, dil=1, subm=False) -> tuple:
    g = make_geom(batch, shape, ksize, stride, pad, dil, subm)
    o = (ctypes.c_int32 * 3)()
    _check(lib().spc_out_shape(ctypes.byref(g), o), "spc_out_shape")
    return tuple(o)


def kmap_workspace(g: Geom, n_in: int) -> int:
    b = ctypes.c_size_t()
    _check(lib().spc_kmap_workspace(ctypes.byref(g), int(n_in), ctypes.byref(b)), "spc_kmap_workspace")
    return b.value


@functools.lru_cache(maxsize=256)
def _kmap_plan(batch, shape, ksize, stride, pad, dil, subm, n_in, table):
    """(Geom, K, workspace bytes) of a kernel-map call; the Geom is shared and
    never modified."""
    g = make_geom(batch, shape, ksize, stride, pad, dil, subm, table)
    return g, int(g.ksize[0] * g.ksize[1] * g.ksize[2]), kmap_workspace(g, n_in)


def strided_out_bound(n_in: int, batch: int, shape, ksize, stride=1, pad=0, dil=1) -> int:
    """Upper bound of a strided map's output-site count that follows from the
    geometry alone (the role of spconv's ``out_inds_num_limit``): along an
    axis the offsets k*dil, k < ksize, reach an exact multiple of the stride at
    most ceil(ksize / (stride / gcd(stride, dil))) times, so an input feeds at
    most the product of those over the axes; and never more than the output
    grid holds."""
    import math
    ks, st, dl = _t3(ksize), _t3(stride), _t3(dil)
    per = 1
    for k, s, d in zip(ks, st, dl):
        per *= -(-k // (s // math.gcd(s, d)))
    vol = int(batch)
    for o in out_shape(batch, shape, ksize, stride, pad, dil, subm=False):
        vol *= max(o, 0)
    return int(min(int(n_in) * per, vol))


def build_kmap(coords: torch.Tensor, batch: int, shape: Sequence[int], ksize, stride=1, pad=0, dil=1,
               subm: bool = True, pairs: bool = True, with_nbr_in: bool = True, orders: bool = False,
               out_cap: Optional[int] = None, workspace: Optional[torch.Tensor] = None,
               table: str = "hash", count_first: bool = False, device_count: bool = False) -> dict:
    """Kernel map of int32 [N, 4] (b, z, y, x) coordinates (spc_build_kmap).

    Returns a dict with ``nbr`` [n_out, K] (submanifold neighbour map or the
    strided output-side map, row-major), ``n_out``, ``coord_err`` (device
    int32 [1]) and, as requested, ``out_coords`` [n_out, 4], ``nbr_in`` [N, K],
    the CSR pair lists ``pair_ptr`` [K+1], ``pair_in`` / ``pair_out`` (first
    pair_ptr[K] entries valid) and the processing orders ``order`` (rows of
    nbr) and ``order_in`` (rows of nbr_in).  A strided call without
    ``out_cap`` sizes its outputs by ``strided_out_bound`` (one library call,
    which returns the count M; the result views hold M rows), or with
    ``count_first`` asks the library for M first and allocates exactly (two
    calls).  ``table`` picks the input table: ``"hash"`` (default) or
    ``"grid"`` (occupancy bitmap + index grid over the whole input grid, 4.125
    bytes of workspace per cell); the results are the same.

    ``device_count`` calls spc_build_kmap_async instead, which never waits:
    the result then holds ``n_out_dev`` (device int32 [1], the row count M in
    stream order), ``n_cap`` (the row capacity, out_cap or the bound) and
    ``n_out`` = None; ``nbr``, ``out_coords`` and ``order`` span n_cap rows,
    of which the first M are valid.  Bad coordinates then show only in
    ``coord_err``, and M > n_cap means the map holds no rows.
    """
    _need(coords, "coords", torch.int32)
    if coords.dim() != 2 or coords.shape[1] != 4:
        raise ValueError("coords must be [N, 4]")
    dev = coords.device
    n = coords.shape[0]
    key = lambda v: v if isinstance(v, int) else tuple(v)
    g, K, ws_bytes = _kmap_plan(int(batch), key(shape), key(ksize), key(stride), key(pad), key(dil), bool(subm), n,
                                table)
    stream = _stream(dev)
    n_out = ctypes.c_int64(0)
    if not subm and out_cap is None and not count_first:
        out_cap = strided_out_bound(n, batch, shape, ksize, stride, pad, dil)
    if device_count and out_cap is None and not subm:
        raise ValueError("device_count needs out_cap (count_first waits for the count)")
    if not subm and out_cap is None:
        ws = workspace if workspace is not None and workspace.numel() >= ws_bytes else \
            torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
        st = lib().spc_build_kmap(ctypes.byref(g), coords.data_ptr(), n, None, 0, ctypes.byref(n_out), None, None,
                                  None, None, None, 0, None, None, None, ws.data_ptr(), ws.numel(), stream)
        _check(st, "spc_build_kmap")
        out_cap = n_out.value
        workspace = ws
    cap = n if subm else int(out_cap)
    # every int32 output in one allocation (each part starts 256-byte aligned)
    # and the workspace in a second one, which the results do not keep alive;
    # the library gets raw addresses, and the result views are made afterwards
    parts = [("err", 4), ("nbr", max(K * cap, 4))]
    if device_count:
        parts.append(("nout", 4))
    if not subm:
        parts.append(("out_coords", max(cap, 1) * 4))
    want_nbr_in = not subm and (with_nbr_in or orders)
    if want_nbr_in:
        parts.append(("nbr_in", max(n * K, 4)))
    if orders:
        parts.append(("order", max(cap, 4)))
        if not subm:
            parts.append(("order_in", max(n, 4)))
    if pairs:
        parts += [("pp", K + 1), ("pi", max(K * n, 4)), ("po", max(K * n, 4))]
    sizes = []
    for _, v in parts:
        sizes += [v, (-v) % 64]
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    buf = torch.empty(sum(sizes), dtype=torch.int32, device=dev)
    base, addr, o = buf.data_ptr(), {}, 0
    for i, (name, _) in enumerate(parts):
        addr[name] = base + 4 * o
        o += sizes[2 * i] + sizes[2 * i + 1]
    a = addr.get
    if device_count:
        st = lib().spc_build_kmap_async(ctypes.byref(g), coords.data_ptr(), n, a("out_coords"), cap, a("nout"),
                                        a("nbr"), a("nbr_in"), a("pp"), a("pi"), a("po"),
                                        max(K * n, 0) if pairs else 0, a("order"), a("order_in"), a("err"),
                                        workspace.data_ptr(), workspace.numel(), stream)
        _check(st, "spc_build_kmap_async")
        m = cap
    else:
        st = lib().spc_build_kmap(ctypes.byref(g), coords.data_ptr(), n, a("out_coords"), cap, ctypes.byref(n_out),
                                  a("nbr"), a("nbr_in"), a("pp"), a("pi"), a("po"), max(K * n, 0) if pairs else 0,
                                  a("order"), a("order_in"), a("err"), workspace.data_ptr(), workspace.numel(), stream)
        _check(st, "spc_build_kmap")
        m = int(n_out.value)
    views = dict(zip((name for name, _ in parts), buf.split_with_sizes(sizes)[0::2]))
    res = {"coord_err": views["err"][:1], "n_out": None if device_count else m, "nbr": views["nbr"][:K * m].view(m, K)}
    if device_count:
        res["n_out_dev"], res["n_cap"] = views["nout"][:1], cap
    if not subm:
        res["out_coords"] = views["out_coords"][:4 * m].view(m, 4)
    if want_nbr_in:
        res["nbr_in"] = views["nbr_in"][:n * K].view(n, K)
    if orders:
        res["order"] = views["order"][:m]
        if not subm:
            res["order_in"] = views["order_in"][:n]
    if pairs:
        res["pair_ptr"], res["pair_in"], res["pair_out"] = views["pp"], views["pi"], views["po"]
    return res


def _conv_checks(x, weight, bias, dev):
    _need(x, "input", dev=dev)
    _need(weight, "weight", x.dtype, dev)
    if x.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {x.dtype}")
    if weight.dim() != 3:
        raise ValueError("weight must be [K, Cin, Cout]")
    if bias is not None:
        _need(bias, "bias", torch.float32, dev)


def _pretranspose(dtype, cin: int, flag) -> bool:
    """Whether a forward hands the kernel pre-transposed weights: for fp32
    and for contractions of more than 64 16-bit channels, where staging W's
    own layout would transpose every offset's weights once per tile (shorter
    16-bit contractions read W's own layout with transposing LDS reads)."""
    if flag is not None:
        return bool(flag)
    return dtype == torch.float32 or cin > 64


def transpose_weight(weight: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """weight [K, cin, cout] -> [K, cout, cin] on the device (spc_transpose_weight)."""
    _need(weight, "weight")
    if weight.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {weight.dtype}")
    if weight.dim() != 3:
        raise ValueError("weight must be [K, Cin, Cout]")
    K, cin, cout = weight.shape
    if out is None:
        out = torch.empty((K, cout, cin), dtype=weight.dtype, device=weight.device)
    else:
        _need(out, "out", weight.dtype, weight.device)
        if tuple(out.shape) != (K, cout, cin):
            raise ValueError(f"out must be [{K}, {cout}, {cin}], got {tuple(out.shape)}")
    st = lib().spc_transpose_weight(_DTYPES[weight.dtype], _ptr(weight), K, cin, cout, _ptr(out),
                                    _stream(weight.device))
    _check(st, "spc_transpose_weight")
    return out


def conv_fwd_wt(feats: torch.Tensor, weight_t: torch.Tensor, bias: Optional[torch.Tensor],
                map_: Optional[torch.Tensor], n_rows: int, map_is_subm: bool = False,
                order: Optional[torch.Tensor] = None, residual: Optional[torch.Tensor] = None,
                relu: bool = False, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Forward with pre-transposed weights weight_t [K, Cout, Cin] (spc_conv_fwd_wt);
    otherwise as conv_fwd_fused."""
    dev = feats.device
    _conv_checks(feats, weight_t, bias, dev)
    for t, nm in ((map_, "map"), (order, "order")):
        if t is not None:
            _need(t, nm, torch.int32, dev)
    K, cout, cin = weight_t.shape
    if residual is not None:
        _need(residual, "residual", feats.dtype, dev)
        if tuple(residual.shape) != (n_rows, cout):
            raise ValueError(f"residual must be [{n_rows}, {cout}], got {tuple(residual.shape)}")
    if out is None:
        out = torch.empty((n_rows, cout), dtype=feats.dtype, device=dev)
    st = lib().spc_conv_fwd_wt(_DTYPES[feats.dtype], _ptr(feats), feats.shape[0], cin, _ptr(weight_t), K, cout,
                               _ptr(bias), _ptr(map_), 1 if map_is_subm else 0, _ptr(order), int(n_rows),
                               _ptr(residual), 1 if relu else 0, _ptr(out), _stream(dev))
    _check(st, "spc_conv_fwd_wt")
    return out


def conv_fwd_dev_rows(feats: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor],
                      map_: torch.Tensor, n_rows_dev: torch.Tensor, row_cap: int,
                      order: Optional[torch.Tensor] = None, weight_t: bool = False,
                      residual: Optional[torch.Tensor] = None, relu: bool = False,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Forward over the rows of a strided map built with device_count
    (spc_conv_fwd_dev_rows): out [row_cap, Cout], of which the first
    n_rows_dev rows are written.  ``weight`` is [K, Cin, Cout], or [K, Cout,
    Cin] from transpose_weight when ``weight_t``."""
    dev = feats.device
    _conv_checks(feats, weight, bias, dev)
    _need(map_, "map", torch.int32, dev)
    _need(n_rows_dev, "n_rows_dev", torch.int32, dev)
    if order is not None:
        _need(order, "order", torch.int32, dev)
    K = weight.shape[0]
    cin, cout = (weight.shape[2], weight.shape[1]) if weight_t else (weight.shape[1], weight.shape[2])
    if residual is not None:
        _need(residual, "residual", feats.dtype, dev)
        if tuple(residual.shape) != (row_cap, cout):
            raise ValueError(f"residual must be [{row_cap}, {cout}], got {tuple(residual.shape)}")
    if out is None:
        out = torch.empty((row_cap, cout), dtype=feats.dtype, device=dev)
    st = lib().spc_conv_fwd_dev_rows(_DTYPES[feats.dtype], _ptr(feats), feats.shape[0], cin, _ptr(weight),
                                     1 if weight_t else 0, K, cout, _ptr(bias), _ptr(map_), _ptr(order),
                                     int(row_cap), _ptr(n_rows_dev), _ptr(residual), 1 if relu else 0, _ptr(out),
                                     _stream(dev))
    _check(st, "spc_conv_fwd_dev_rows")
    return out


def subm_conv_fwd(feats: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor],
                  nbr: Optional[torch.Tensor], order: Optional[torch.Tensor] = None,
                  out: Optional[torch.Tensor] = None, pretranspose: Optional[bool] = None) -> torch.Tensor:
    """out[c] = bias + sum_k feats[nbr[c, k]] @ W[k] (spc_subm_conv_fwd, or
    spc_transpose_weight + spc_conv_fwd_wt when `pretranspose`, by default
    for fp32 and Cin > 64: the same result bit for bit)."""
    dev = feats.device
    _conv_checks(feats, weight, bias, dev)
    K, cin, cout = weight.shape
    n = feats.shape[0]
    for t, nm in ((nbr, "nbr"), (order, "order")):
        if t is not None:
            _need(t, nm, torch.int32, dev)
    if _pretranspose(feats.dtype, cin, pretranspose):
        if K > 1 and nbr is None:
            raise ValueError("nbr is required for K > 1")
        return conv_fwd_wt(feats, transpose_weight(weight), bias, nbr if K > 1 else None, n, K > 1,
                           order if K > 1 else None, out=out)
    if out is None:
        out = torch.empty((n, cout), dtype=feats.dtype, device=dev)
    st = lib().spc_subm_conv_fwd(_DTYPES[feats.dtype], _ptr(feats), n, cin, _ptr(weight), K, cout, _ptr(bias),
                                 _ptr(nbr), _ptr(order), _ptr(out), _stream(dev))
    _check(st, "spc_subm_conv_fwd")
    return out


def sparse_conv_fwd(feats: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor],
                    nbr_out: torch.Tensor, n_out: int, order: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, pretranspose: Optional[bool] = None) -> torch.Tensor:
    """Strided forward over the n_out output rows of a strided kernel map
    (spc_sparse_conv_fwd; `pretranspose` as for subm_conv_fwd)."""
    dev = feats.device
    _conv_checks(feats, weight, bias, dev)
    _need(nbr_out, "nbr_out", torch.int32, dev)
    if order is not None:
        _need(order, "order", torch.int32, dev)
    K, cin, cout = weight.shape
    if _pretranspose(feats.dtype, cin, pretranspose):
        return conv_fwd_wt(feats, transpose_weight(weight), bias, nbr_out, n_out, False, order, out=out)
    if out is None:
        out = torch.empty((n_out, cout), dtype=feats.dtype, device=dev)
    st = lib().spc_sparse_conv_fwd(_DTYPES[feats.dtype], _ptr(feats), feats.shape[0], cin, _ptr(weight), K, cout,
                                   _ptr(bias), _ptr(nbr_out), _ptr(order), int(n_out), _ptr(out), _stream(dev))
    _check(st, "spc_sparse_conv_fwd")
    return out


def sparse_inverse_conv_fwd(feats: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor],
                            nbr_in: torch.Tensor, n_fine: int, order_in: Optional[torch.Tensor] = None,
                            out: Optional[torch.Tensor] = None,
                            pretranspose: Optional[bool] = None) -> torch.Tensor:
    """Inverse (upsampling) forward onto the input sites of a strided kernel map
    (spc_sparse_inverse_conv_fwd): feats [n_coarse, cin] -> [n_fine, cout];
    `pretranspose` as for subm_conv_fwd."""
    dev = feats.device
    _conv_checks(feats, weight, bias, dev)
    _need(nbr_in, "nbr_in", torch.int32, dev)
    if order_in is not None:
        _need(order_in, "order_in", torch.int32, dev)
    K, cin, cout = weight.shape
    if _pretranspose(feats.dtype, cin, pretranspose):
        return conv_fwd_wt(feats, transpose_weight(weight), bias, nbr_in, n_fine, False, order_in, out=out)
    if out is None:
        out = torch.empty((n_fine, cout), dtype=feats.dtype, device=dev)
    st = lib().spc_sparse_inverse_conv_fwd(_DTYPES[feats.dtype], _ptr(feats), feats.shape[0], cin, _ptr(weight), K,
                                           cout, _ptr(bias), _ptr(nbr_in), _ptr(order_in), int(n_fine), _ptr(out),
                                           _stream(dev))
    _check(st, "spc_sparse_inverse_conv_fwd")
    return out


def conv_fwd_fused(feats: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor],
                   map_: Optional[torch.Tensor], n_rows: int, order: Optional[torch.Tensor] = None,
                   residual: Optional[torch.Tensor] = None, relu: bool = False,
                   out: Optional[torch.Tensor] = None, pretranspose: Optional[bool] = None) -> torch.Tensor:
    """Forward over any map with the fused bias + residual + ReLU epilogue
    (spc_conv_fwd_fused); ``out`` may be ``residual`` itself; `pretranspose`
    as for subm_conv_fwd."""
    dev = feats.device
    _conv_checks(feats, weight, bias, dev)
    for t, nm in ((map_, "map"), (order, "order")):
        if t is not None:
            _need(t, nm, torch.int32, dev)
    K, cin, cout = weight.shape
    if residual is not None:
        _need(residual, "residual", feats.dtype, dev)
        if tuple(residual.shape) != (n_rows, cout):
            raise ValueError(f"residual must be [{n_rows}, {cout}], got {tuple(residual.shape)}")
    if _pretranspose(feats.dtype, cin, pretranspose):
        return conv_fwd_wt(feats, transpose_weight(weight), bias, map_, n_rows, False, order, residual, relu, out)
    if out is None:
        out = torch.empty((n_rows, cout), dtype=feats.dtype, device=dev)
    st = lib().spc_conv_fwd_fused(_DTYPES[feats.dtype], _ptr(feats), feats.shape[0], cin, _ptr(weight), K, cout,
                                  _ptr(bias), _ptr(map_), _ptr(order), int(n_rows), _ptr(residual),
                                  1 if relu else 0, _ptr(out), _stream(dev))
    _check(st, "spc_conv_fwd_fused")
    return out


def conv_bwd_input(dout: torch.Tensor, weight: torch.Tensor, map_: Optional[torch.Tensor], map_is_subm: bool,
                   n_in: int, order: Optional[torch.Tensor] = None,
                   din: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Gradient of the input features (spc_conv_bwd_input)."""
    dev = dout.device
    _conv_checks(dout, weight, None, dev)
    for t, nm in ((map_, "map"), (order, "order")):
        if t is not None:
            _need(t, nm, torch.int32, dev)
    K, cin, cout = weight.shape
    if din is None:
        din = torch.empty((n_in, cin), dtype=dout.dtype, device=dev)
    st = lib().spc_conv_bwd_input(_DTYPES[dout.dtype], _ptr(dout), dout.shape[0], cout, _ptr(weight), K, cin,
                                  _ptr(map_), 1 if map_is_subm else 0, _ptr(order), int(n_in), _ptr(din),
                                  _stream(dev))
    _check(st, "spc_conv_bwd_input")
    return din


@functools.lru_cache(maxsize=256)
def conv_bwd_filter_workspace(n_in, n_out, cin, cout, K, want_dbias) -> int:
    b = ctypes.c_size_t()
    _check(lib().spc_conv_bwd_filter_workspace(int(n_in), int(n_out), int(cin), int(cout), int(K),
                                               1 if want_dbias else 0, ctypes.byref(b)),
           "spc_conv_bwd_filter_workspace")
    return b.value


def conv_bwd_filter(feats: torch.Tensor, dout: torch.Tensor, K: int, pair_ptr: Optional[torch.Tensor],
                    pair_in: Optional[torch.Tensor], pair_out: Optional[torch.Tensor], want_dbias: bool = False,
                    workspace: Optional[torch.Tensor] = None, dw: Optional[torch.Tensor] = None):
    """Weight (and optionally bias) gradient from CSR pair lists (spc_conv_bwd_filter).

    Returns ``(dw [K, Cin, Cout] fp32, dbias [Cout] fp32 or None)``."""
    dev = feats.device
    _need(feats, "feats", dev=dev)
    _need(dout, "dout", feats.dtype, dev)
    for t, nm in ((pair_ptr, "pair_ptr"), (pair_in, "pair_in"), (pair_out, "pair_out")):
        if t is not None:
            _need(t, nm, torch.int32, dev)
    cin, cout = feats.shape[1], dout.shape[1]
    ws = conv_bwd_filter_workspace(feats.shape[0], dout.shape[0], cin, cout, int(K), bool(want_dbias))
    if workspace is None or workspace.numel() < ws:
        workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
    if dw is None:
        dw = torch.empty((K, cin, cout), dtype=torch.float32, device=dev)
    db = torch.empty(cout, dtype=torch.float32, device=dev) if want_dbias else None
    st = lib().spc_conv_bwd_filter(_DTYPES[feats.dtype], _ptr(feats), feats.shape[0], cin, _ptr(dout),
                                   dout.shape[0], cout, int(K), _ptr(pair_ptr), _ptr(pair_in), _ptr(pair_out),
                                   _ptr(dw), _ptr(db), _ptr(workspace), workspace.numel(), _stream(dev))
    _check(st, "spc_conv_bwd_filter")
    return dw, db


def conv_bwd_filter_noalloc(feats: torch.Tensor, dout: torch.Tensor, K: int, pair_ptr: Optional[torch.Tensor],
                            pair_in: Optional[torch.Tensor], pair_out: Optional[torch.Tensor], dw: torch.Tensor,
                            dbias: Optional[torch.Tensor] = None) -> None:
    """spc_conv_bwd_filter_noalloc: the weight (and optionally bias) gradient
    into the caller's ``dw`` [K, Cin, Cout] fp32 (and ``dbias`` [Cout] fp32),
    with the library's static scratch instead of a workspace; neither the
    binding nor the library allocates anything."""
    dev = feats.device
    _need(feats, "feats", dev=dev)
    _need(dout, "dout", feats.dtype, dev)
    for t, nm in ((pair_ptr, "pair_ptr"), (pair_in, "pair_in"), (pair_out, "pair_out")):
        if t is not None:
            _need(t, nm, torch.int32, dev)
    cin, cout = feats.shape[1], dout.shape[1]
    _need(dw, "dw", torch.float32, dev)
    if tuple(dw.shape) != (int(K), cin, cout):
        raise ValueError(f"dw must be [{K}, {cin}, {cout}], got {tuple(dw.shape)}")
    if dbias is not None:
        _need(dbias, "dbias", torch.float32, dev)
        if tuple(dbias.shape) != (cout,):
            raise ValueError(f"dbias must be [{cout}], got {tuple(dbias.shape)}")
    st = lib().spc_conv_bwd_filter_noalloc(_DTYPES[feats.dtype], _ptr(feats), feats.shape[0], cin, _ptr(dout),
                                           dout.shape[0], cout, int(K), _ptr(pair_ptr), _ptr(pair_in),
                                           _ptr(pair_out), _ptr(dw), _ptr(dbias), _stream(dev))
    _check(st, "spc_conv_bwd_filter_noalloc")


def sparse_maxpool_fwd(feats: torch.Tensor, nbr_out: torch.Tensor, n_out: int, want_argk: bool = True,
                       out: Optional[torch.Tensor] = None, argk: Optional[torch.Tensor] = None):
    """Channel-wise max over each output's map row (spc_sparse_maxpool_fwd):
    returns ``(out [n_out, C], argk uint8 [n_out, C] or None)``."""
    dev = feats.device
    _need(feats, "feats", feats.dtype, dev)
    _need(nbr_out, "nbr_out", torch.int32, dev)
    C = feats.shape[1]
    K = nbr_out.shape[1] if nbr_out.dim() == 2 else 0
    if out is None:
        out = torch.empty((n_out, C), dtype=feats.dtype, device=dev)
    if want_argk and argk is None:
        argk = torch.empty((n_out, C), dtype=torch.uint8, device=dev)
    st = lib().spc_sparse_maxpool_fwd(_DTYPES[feats.dtype], _ptr(feats), feats.shape[0], C, _ptr(nbr_out), K,
                                      int(n_out), _ptr(out), _ptr(argk if want_argk else None), _stream(dev))
    _check(st, "spc_sparse_maxpool_fwd")
    return out, (argk if want_argk else None)


def sparse_maxpool_bwd(dout: torch.Tensor, argk: torch.Tensor, nbr_in: torch.Tensor, n_in: int,
                       din: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Gradient of the pooled features routed to the winning inputs (spc_sparse_maxpool_bwd)."""
    dev = dout.device
    _need(dout, "dout", dout.dtype, dev)
    _need(argk, "argk", torch.uint8, dev)
    _need(nbr_in, "nbr_in", torch.int32, dev)
    C = dout.shape[1]
    K = nbr_in.shape[1] if nbr_in.dim() == 2 else 0
    if din is None:
        din = torch.empty((n_in, C), dtype=dout.dtype, device=dev)
    st = lib().spc_sparse_maxpool_bwd(_DTYPES[dout.dtype], _ptr(dout), dout.shape[0], C, _ptr(argk), _ptr(nbr_in),
                                      K, int(n_in), _ptr(din), _stream(dev))
    _check(st, "spc_sparse_maxpool_bwd")
    return din


def point_to_voxel(points: torch.Tensor, vsize_xyz, coors_range_xyz, max_num_voxels: int,
                   max_num_points_per_voxel: int, empty_mean: bool = True, with_id: bool = False):
    """Voxelise a point cloud [N, F] fp32 (spc_point_to_voxel), like spconv's
    PointToVoxel: returns (voxels [V, P, F], coords [V, 3] ZYX, num_points [V])
    and, with ``with_id``, the per-point voxel ids [N] as a fourth item."""
    dev = points.device
    _need(points, "points", torch.float32, dev)
    if points.dim() != 2:
        raise ValueError("points must be [N, F]")
    n, F = points.shape
    vs = (ctypes.c_float * 3)(*[float(v) for v in vsize_xyz])
    rg = (ctypes.c_float * 6)(*[float(v) for v in coors_range_xyz])
    b = ctypes.c_size_t()
    _check(lib().spc_point_to_voxel_workspace(n, F, int(max_num_voxels), int(max_num_points_per_voxel),
                                              ctypes.byref(b)), "spc_point_to_voxel_workspace")
    ws = torch.empty(max(int(b.value), 16), dtype=torch.uint8, device=dev)
    voxels = torch.empty((max_num_voxels, max_num_points_per_voxel, F), dtype=torch.float32, device=dev)
    coords = torch.empty((max_num_voxels, 3), dtype=torch.int32, device=dev)
    num = torch.empty((max_num_voxels,), dtype=torch.int32, device=dev)
    pcid = torch.empty((n,), dtype=torch.int32, device=dev) if with_id else None
    nv = ctypes.c_int64()
    st = lib().spc_point_to_voxel(_ptr(points), n, F, vs, rg, int(max_num_voxels), int(max_num_points_per_voxel),
                                  1 if empty_mean else 0, _ptr(voxels), _ptr(coords), _ptr(num), _ptr(pcid),
                                  ctypes.byref(nv), _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "spc_point_to_voxel")
    V = nv.value
    res = (voxels[:V], coords[:V], num[:V])
    return res + (pcid,) if with_id else res


def gather_by_voxel_id(seg_features: torch.Tensor, pc_voxel_id: torch.Tensor,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-point features from per-voxel ones, zeros for id -1 (spc_gather_by_voxel_id)."""
    dev = seg_features.device
    _need(seg_features, "seg_features", seg_features.dtype, dev)
    _need(pc_voxel_id, "pc_voxel_id", torch.int32, dev)
    C = seg_features.shape[1]
    if out is None:
        out = torch.empty((pc_voxel_id.shape[0], C), dtype=seg_features.dtype, device=dev)
    st = lib().spc_gather_by_voxel_id(_DTYPES[seg_features.dtype], _ptr(seg_features), seg_features.shape[0], C,
                                      _ptr(pc_voxel_id), pc_voxel_id.shape[0], _ptr(out), _stream(dev))
    _check(st, "spc_gather_by_voxel_id")
    return out


def calibrate_mfma(shape: int, blocks: int, iters: int, sink: torch.Tensor) -> float:
    """Launches the MFMA rate probe (spc_calibrate_mfma) on the current stream
    and returns the FLOP it executes; the caller times it."""
    _need(sink, "sink", torch.float32)
    if sink.numel() < blocks * 256:
        raise ValueError("sink needs blocks * 256 floats")
    f = ctypes.c_double(0.0)
    _check(lib().spc_calibrate_mfma(int(shape), int(blocks), int(iters), _ptr(sink), ctypes.byref(f),
                                    _stream(sink.device)), "spc_calibrate_mfma")
    return f.value
