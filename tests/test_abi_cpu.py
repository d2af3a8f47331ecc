"""The C ABI without a GPU: the library loads, exports every function that
include/spc.h declares, and host-side checks return their status before any
launch (so fake, never-dereferenced pointers are safe here)."""

import ctypes
import os
import re

import pytest

import sparse_convolution_hash_amd.binding as B
from oracle import kmap as O

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "spc.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="libspc.so not built")

FAKE = ctypes.c_void_p(0x100000)        # 16-byte aligned, never dereferenced
MISALIGNED = ctypes.c_void_p(0x100008)


def declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:spc_status|const char\*)\s+(spc_\w+)\(", txt, re.M)))


def test_header_declares_the_boundary():
    names = declared()
    for f in ("spc_build_kmap", "spc_subm_conv_fwd", "spc_sparse_conv_fwd", "spc_conv_bwd_input",
              "spc_conv_bwd_filter"):
        assert f in names
    assert sorted(B.EXPORTS) == names


def test_every_declared_symbol_is_exported():
    L = B.lib()
    for name in declared():
        assert hasattr(L, name), name
    assert B.version().startswith("libspc")


@pytest.mark.parametrize("shape,k,s,p,d", [
    ((41, 1600, 1408), 3, 2, 1, 1), ((8, 200, 200), 3, 2, (0, 1, 1), 1), ((10, 11, 12), 2, 3, 0, 2),
    ((5, 5, 5), 3, 1, 0, 3), ((3, 3, 3), 5, 2, 0, 1),
])
def test_out_shape_matches_oracle(shape, k, s, p, d):
    assert B.out_shape(1, shape, k, s, p, d, subm=False) == O.out_shape(shape, k, s, p, d)


def _ws(g, n):
    b = ctypes.c_size_t()
    return B.lib().spc_kmap_workspace(ctypes.byref(g), n, ctypes.byref(b)), b.value


def test_kmap_workspace_checks():
    assert _ws(B.make_geom(2, (41, 1600, 1408), 3), 120000)[0] == B.SPC_OK
    assert _ws(B.make_geom(1, (8, 8, 8), 2), 10)[0] == B.SPC_ERR_ARG            # even submanifold k
    assert _ws(B.make_geom(0, (8, 8, 8), 3), 10)[0] == B.SPC_ERR_ARG            # batch
    assert _ws(B.make_geom(1, (0, 8, 8), 3), 10)[0] == B.SPC_ERR_ARG            # shape
    assert _ws(B.make_geom(64, (2048, 2048, 1024), 3), 10)[0] == B.SPC_ERR_UNSUPPORTED  # key space
    assert _ws(B.make_geom(1, (8, 8, 8), 9), 10)[0] == B.SPC_ERR_UNSUPPORTED    # ksize > 7
    assert _ws(B.make_geom(1, (8, 8, 8), 3, 0, 1, 1, subm=False), 10)[0] == B.SPC_ERR_ARG  # stride 0
    assert _ws(B.make_geom(1, (8, 8, 8), 3), -1)[0] == B.SPC_ERR_ARG
    st, small = _ws(B.make_geom(1, (8, 8, 8), 3), 10)
    st2, big = _ws(B.make_geom(1, (8, 8, 8), 3), 100000)
    assert st == st2 == B.SPC_OK and big > small


def test_build_kmap_host_checks():
    L = B.lib()
    g = B.make_geom(1, (8, 8, 8), 3)
    n_out = ctypes.c_int64()
    args = lambda **kw: dict(dict(coords=FAKE, nbr=FAKE, pp=None, pi=None, po=None, cap=0, ws=FAKE, wsb=1 << 30), **kw)

    def call(**kw):
        a = args(**kw)
        return L.spc_build_kmap(ctypes.byref(g), a["coords"], 10, None, 0, ctypes.byref(n_out), a["nbr"], None,
                                a["pp"], a["pi"], a["po"], a["cap"], None, a.get("order_in"), None, a["ws"],
                                a["wsb"], None)
    assert call(ws=None) == B.SPC_ERR_ARG
    assert call(wsb=16) == B.SPC_ERR_WORKSPACE
    assert call(coords=None) == B.SPC_ERR_ARG
    assert call(nbr=None) == B.SPC_ERR_ARG
    assert call(coords=MISALIGNED) == B.SPC_ERR_ARG
    assert call(pp=FAKE) == B.SPC_ERR_ARG                       # pair lists: all or none
    assert call(pp=FAKE, pi=FAKE, po=FAKE, cap=10) == B.SPC_ERR_ARG  # pair_cap < K * n
    assert "pair_cap" in B.lib().spc_last_error().decode()
    assert call(order_in=FAKE) == B.SPC_ERR_ARG                 # order_in is for strided maps


def test_conv_host_checks():
    L = B.lib()
    fwd = lambda dt, cin, cout, K, nbr=FAKE, x=FAKE: L.spc_subm_conv_fwd(dt, x, 100, cin, FAKE, K, cout, None,
                                                                        nbr, None, FAKE, None)
    assert fwd(2, 24, 32, 27) == B.SPC_ERR_UNSUPPORTED          # cin not a multiple of 16
    assert fwd(2, 32, 8, 27) == B.SPC_ERR_UNSUPPORTED
    assert fwd(7, 32, 32, 27) == B.SPC_ERR_ARG                  # dtype
    assert fwd(2, 32, 32, 0) == B.SPC_ERR_ARG                   # K
    assert fwd(2, 32, 32, 27, nbr=None) == B.SPC_ERR_ARG        # map required for K > 1
    assert fwd(2, 32, 32, 27, x=MISALIGNED) == B.SPC_ERR_ARG
    # zero rows: valid, nothing launched
    assert L.spc_subm_conv_fwd(2, None, 0, 32, FAKE, 27, 32, None, None, None, FAKE, None) == B.SPC_OK
    # submanifold dinput needs n_out == n_in
    assert L.spc_conv_bwd_input(1, FAKE, 10, 64, FAKE, 27, 64, FAKE, 1, None, 11, FAKE, None) == B.SPC_ERR_ARG
    assert L.spc_subm_conv_fwd(2, FAKE, 100, 32, FAKE, 27, 32, None, FAKE, MISALIGNED, FAKE, None) == B.SPC_ERR_ARG
    b = ctypes.c_size_t()
    assert L.spc_conv_bwd_filter_workspace(1000, 1000, 64, 64, 27, 1, ctypes.byref(b)) == B.SPC_OK and b.value > 0
    # dfilter: identity pairs only for K == 1, workspace size enforced
    assert L.spc_conv_bwd_filter(1, FAKE, 10, 64, FAKE, 10, 64, 27, None, None, None, FAKE, None, FAKE,
                                 1 << 30, None) == B.SPC_ERR_ARG
    assert L.spc_conv_bwd_filter(1, FAKE, 10, 64, FAKE, 10, 64, 1, None, None, None, FAKE, None, FAKE,
                                 8, None) == B.SPC_ERR_WORKSPACE


def test_pretransposed_forward_host_checks():
    L = B.lib()
    tw = lambda dt, K, cin, cout, w=FAKE, wt=ctypes.c_void_p(0x200000): L.spc_transpose_weight(dt, w, K, cin, cout,
                                                                                              wt, None)
    assert tw(7, 27, 16, 16) == B.SPC_ERR_ARG                   # dtype
    assert tw(2, 0, 16, 16) == B.SPC_ERR_ARG                    # K
    assert tw(2, 27, 0, 16) == B.SPC_ERR_ARG                    # cin
    assert tw(2, 27, 16, 16, w=None) == B.SPC_ERR_ARG
    assert tw(2, 27, 256, 256) == B.SPC_ERR_ARG                 # 0x100000 + 3.5 MB overlaps 0x200000
    assert "overlap" in L.spc_last_error().decode()
    fwd = lambda dt, cin, cout, K, m=FAKE, n_src=100, n_rows=100: L.spc_conv_fwd_wt(
        dt, FAKE, n_src, cin, FAKE, K, cout, None, m, 1, None, n_rows, None, 0, FAKE, None)
    assert fwd(2, 24, 32, 27) == B.SPC_ERR_UNSUPPORTED          # cin not a multiple of 16
    assert fwd(7, 32, 32, 27) == B.SPC_ERR_ARG                  # dtype
    assert fwd(2, 32, 32, 27, m=None) == B.SPC_ERR_ARG          # map required for K > 1
    assert fwd(2, 32, 32, 1, m=None, n_src=10) == B.SPC_ERR_ARG  # identity needs n_src == n_rows
    assert fwd(2, 32, 32, 27, n_rows=0) == B.SPC_OK             # zero rows: nothing launched


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(TypeError):
        B.subm_conv_fwd(torch.zeros(4, 16), torch.zeros(27, 16, 16), None, torch.zeros(27, 4, dtype=torch.int32))


def test_kmap_table_choice():
    # the hash (default) needs 2^ceil(log2 4N) 8-byte slots; the index grid
    # 4 bytes per cell plus a bit per cell; any other table value is refused
    lidar = dict(batch=2, shape=(41, 1600, 1408), ksize=3)
    st, hash_bytes = _ws(B.make_geom(**lidar), 120000)
    st2, grid_bytes = _ws(B.make_geom(**lidar, table="grid"), 120000)
    cells = 2 * 41 * 1600 * 1408
    assert st == st2 == B.SPC_OK
    assert hash_bytes >= (1 << 19) * 8 and hash_bytes < 64 << 20
    assert grid_bytes >= cells * 4 + cells // 8
    g = B.make_geom(**lidar)
    g.table = 2
    assert _ws(g, 120000)[0] == B.SPC_ERR_ARG
    assert "table" in B.lib().spc_last_error().decode()
    with pytest.raises(ValueError):
        B.make_geom(**lidar, table="dense")


@pytest.mark.parametrize("shape,k,s,p,d", [
    ((7, 8, 6), 3, 2, 1, 1), ((8, 8, 8), 2, 2, 0, 1), ((9, 7, 8), 3, 1, 0, 2), ((8, 9, 7), 3, 3, 2, 1),
    ((12, 12, 12), 5, 2, 2, 1), ((10, 10, 10), 3, 2, 1, 2),
])
def test_strided_out_bound_holds(shape, k, s, p, d):
    # the geometric bound the binding sizes strided outputs by is never below
    # the oracle's output count, and equals 8N for k3 s2 on a large grid
    import workloads as W
    c = W.tiny_grid(W.rng(400 + k * s), min(shape), 0.3, 2)
    m = O.strided_kmap(c, 2, shape, k, s, p, d)["out_coords"].shape[0]
    assert m <= B.strided_out_bound(c.shape[0], 2, shape, k, s, p, d)
    assert B.strided_out_bound(1000, 2, (41, 1600, 1408), 3, 2, 1, 1) == 8000
    assert B.strided_out_bound(10 ** 7, 1, (8, 8, 8), 3, 2, 1, 1) == 4 * 4 * 4


def test_noalloc_dfilter_host_checks():
    # the allocation-free dfilter refuses, before any HIP call, sizes whose
    # scratch exceeds its static array, and bad arguments as the workspace form
    L = B.lib()
    call = lambda cin, cout, K, pp=FAKE, x=FAKE: L.spc_conv_bwd_filter_noalloc(
        2, x, 100, cin, FAKE, 100, cout, K, pp, FAKE, FAKE, FAKE, None, None)
    assert call(256, 256, 27) == B.SPC_ERR_UNSUPPORTED
    assert "scratch" in L.spc_last_error().decode()
    assert call(128, 128, 125) == B.SPC_ERR_UNSUPPORTED
    assert call(24, 32, 27) == B.SPC_ERR_UNSUPPORTED              # channels not multiples of 16
    assert call(128, 128, 27, x=MISALIGNED) == B.SPC_ERR_ARG
    assert call(128, 128, 27, pp=None) == B.SPC_ERR_ARG            # pair lists: all or none
    b = ctypes.c_size_t()
    assert L.spc_conv_bwd_filter_workspace(10 ** 6, 10 ** 6, 128, 128, 27, 1, ctypes.byref(b)) == B.SPC_OK
    assert b.value <= 36 << 20                                     # the named workloads' largest layer fits


def test_calibrate_mfma_host_checks():
    L = B.lib()
    assert L.spc_calibrate_mfma(2, 256, 10, FAKE, None, None) == B.SPC_ERR_ARG      # shape
    assert L.spc_calibrate_mfma(0, 0, 10, FAKE, None, None) == B.SPC_ERR_ARG        # blocks
    assert L.spc_calibrate_mfma(1, 256, 10, None, None, None) == B.SPC_ERR_ARG      # sink


def test_async_kmap_and_dev_rows_host_checks():
    # the forms that leave the row count in device memory check their extra
    # arguments before any HIP call
    L = B.lib()
    g = B.make_geom(2, (41, 1600, 1408), 3, 2, 1, 1, subm=False)
    call = lambda out_coords=FAKE, n_out_dev=FAKE, ws=FAKE: L.spc_build_kmap_async(
        ctypes.byref(g), FAKE, 1000, out_coords, 8000, n_out_dev, FAKE, None, None, None, None, 0, None, None,
        FAKE, ws, 1 << 20, None)
    assert call(n_out_dev=None) == B.SPC_ERR_ARG
    assert "n_out_dev" in L.spc_last_error().decode()
    assert call(out_coords=None) == B.SPC_ERR_ARG                   # no count-only form
    assert call(n_out_dev=MISALIGNED) == B.SPC_ERR_ARG
    assert call(ws=FAKE) == B.SPC_ERR_WORKSPACE                     # 1 MiB is short of this map's workspace
    fwd = lambda n_rows_dev=FAKE, cin=64, cap=100: L.spc_conv_fwd_dev_rows(
        1, FAKE, 100, cin, FAKE, 0, 27, 64, None, FAKE, None, cap, n_rows_dev, None, 0, FAKE, None)
    assert fwd(n_rows_dev=None) == B.SPC_ERR_ARG
    assert fwd(n_rows_dev=MISALIGNED) == B.SPC_ERR_ARG
    assert fwd(cin=24) == B.SPC_ERR_UNSUPPORTED
    assert fwd(cap=-1) == B.SPC_ERR_ARG
