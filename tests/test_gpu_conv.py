"""GPU convolutions vs the oracle (fp64): submanifold and strided forward,
k=1, dinput, dfilter and dbias, for fp32 / fp16 / bf16, at small sizes that
span several tiles with ragged tails and at the named workloads' full sizes."""

import numpy as np
import pytest
import torch

import sparse_convolution_hash_amd as spc
import workloads as W
from oracle import conv as OC
from oracle import kmap as O
from tests.parity import TOL, TOL_DW, assert_close, cuda, host, hygon_check

pytestmark = pytest.mark.gpu

DTYPES = [torch.float32, torch.float16, torch.bfloat16]


def _subm_case(seed, side, fill, batch, k, cin, cout, dtype, bias=True):
    c = W.tiny_grid(W.rng(seed), side, fill, batch)
    t = W.small_layer(seed, c, cin, cout, k ** 3, dtype, bias=bias)
    return c, t


def run_subm_layer(c, batch, shape, k, t, dtype, train=True, what="", ordered=True):
    """Forward (and dinput / dfilter / dbias) of one submanifold layer vs the oracle."""
    print(f"subm conv {what} n={c.shape[0]} k={k} {tuple(t['weight'].shape)} {dtype} ordered={ordered}", flush=True)
    km = spc.build_kmap(cuda(c), batch, shape, k, pairs=train, orders=ordered)
    nbr_ref = O.subm_kmap(c, shape, k)
    x, w = cuda(t["feats"]), cuda(t["weight"])
    b = cuda(t["bias"]) if t.get("bias") is not None else None
    order = km.get("order") if k > 1 else None
    out = spc.subm_conv_fwd(x, w, b, km["nbr"] if k > 1 else None, order)
    errs = {"fwd": assert_close(out, OC.conv_fwd(t["feats"], t["weight"], t["bias"], nbr_ref), TOL[dtype], "fwd")}
    if not train:
        return errs
    g = cuda(t["grad"])
    din = spc.conv_bwd_input(g, w, km["nbr"] if k > 1 else None, True, c.shape[0], order)
    errs["din"] = assert_close(din, OC.conv_bwd_input(t["grad"], t["weight"], nbr_ref, c.shape[0]), TOL[dtype], "din")
    pp, pi, po = (km["pair_ptr"], km["pair_in"], km["pair_out"]) if k > 1 else (None, None, None)
    dw, db = spc.conv_bwd_filter(x, g, k ** 3, pp, pi, po, want_dbias=True)
    errs["dw"] = assert_close(dw, OC.conv_bwd_filter(t["feats"], t["grad"], nbr_ref), TOL_DW, "dw")
    errs["db"] = assert_close(db, OC.conv_bwd_bias(t["grad"]), TOL_DW, "dbias")
    if what:  # the named workloads: the Hygon README's acceptance test as well
        cin, cout = t["weight"].shape[1], t["weight"].shape[2]
        fp32 = dtype == torch.float32
        hygon_check(out, OC.conv_fwd(t["feats"], t["weight"], t["bias"], nbr_ref), cin, cout, fp32, "fwd")
        hygon_check(din, OC.conv_bwd_input(t["grad"], t["weight"], nbr_ref, c.shape[0]), cin, cout, fp32, "din")
        hygon_check(dw, OC.conv_bwd_filter(t["feats"], t["grad"], nbr_ref), cin, cout, fp32, "dw")
    return errs


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("seed,side,fill,batch,k,cin,cout", [
    (1, 9, 0.3, 1, 3, 16, 16),        # one tile, ragged
    (2, 14, 0.25, 2, 3, 32, 48),      # several tiles, cout 48 (3 blocks)
    (3, 12, 0.4, 1, 3, 64, 128),      # full 128-channel tile
    (4, 10, 0.3, 2, 1, 48, 32),       # k = 1 (identity map)
    (5, 8, 0.5, 1, 5, 16, 32),        # k = 5, 125 offsets (several offset tiles)
    (6, 16, 0.2, 3, 3, 96, 96),
    (7, 11, 0.3, 1, 3, 144, 32),      # contraction above 128 channels
])
def test_subm_small(dtype, seed, side, fill, batch, k, cin, cout):
    if dtype == torch.float32 and cin > 128:
        pytest.skip("fp32 contraction is limited to 128 channels")
    c, t = _subm_case(seed, side, fill, batch, k, cin, cout, dtype)
    run_subm_layer(c, batch, (side,) * 3, k, t, dtype, ordered=seed % 2 == 1)


@pytest.mark.parametrize("dtype", DTYPES)
def test_single_voxel_and_empty(dtype):
    c = np.array([[0, 1, 2, 3]], np.int32)
    t = W.small_layer(3, c, 16, 32, 27, dtype)
    run_subm_layer(c, 1, (4, 4, 4), 3, t, dtype)
    out = spc.subm_conv_fwd(cuda(t["feats"][:0]), cuda(t["weight"]), None,
                            torch.empty((0, 27), dtype=torch.int32, device="cuda"))
    assert out.shape == (0, 32)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape,k,s,p,d,cin,cout", [
    ((12, 14, 10), 3, 2, 1, 1, 16, 32), ((15, 13, 11), 2, 2, 0, 1, 32, 16), ((11, 11, 11), 3, 1, 0, 2, 48, 64),
])
def test_strided_small(dtype, shape, k, s, p, d, cin, cout):
    c = W.tiny_grid(W.rng(40 + k + s), min(shape), 0.25, 2)
    print(f"strided conv n={c.shape[0]} {shape} k={k} s={s} {dtype}", flush=True)
    km = spc.build_kmap(cuda(c), 2, shape, k, s, p, d, subm=False, orders=True)
    ref = O.strided_kmap(c, 2, shape, k, s, p, d)
    M = ref["out_coords"].shape[0]
    t = W.small_layer(50, c, cin, cout, k ** 3, dtype, n_out=M)
    x, w, b, g = cuda(t["feats"]), cuda(t["weight"]), cuda(t["bias"]), cuda(t["grad"])
    out = spc.sparse_conv_fwd(x, w, b, km["nbr"], km["n_out"], km["order"])
    assert_close(out, OC.conv_fwd(t["feats"], t["weight"], t["bias"], ref["nbr_out"]), TOL[dtype], "fwd")
    out2 = spc.sparse_conv_fwd(x, w, b, km["nbr"], km["n_out"])
    assert torch.equal(out, out2)          # the processing order never changes a result
    din = spc.conv_bwd_input(g, w, km["nbr_in"], False, c.shape[0], km["order_in"])
    assert_close(din, OC.conv_bwd_input(t["grad"], t["weight"], ref["nbr_out"], c.shape[0]), TOL[dtype], "din")
    dw, db = spc.conv_bwd_filter(x, g, k ** 3, km["pair_ptr"], km["pair_in"], km["pair_out"], want_dbias=True)
    assert_close(dw, OC.conv_bwd_filter(t["feats"], t["grad"], ref["nbr_out"]), TOL_DW, "dw")
    assert_close(db, OC.conv_bwd_bias(t["grad"]), TOL_DW, "dbias")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("seed,cin,cout,k", [(11, 128, 128, 3), (12, 96, 64, 3), (13, 144, 32, 1), (14, 32, 48, 3)])
def test_pretransposed_weights_bit_identical(dtype, seed, cin, cout, k):
    """Pre-transposed weights (spc_transpose_weight + spc_conv_fwd_wt) stage the
    same LDS slabs as the per-tile transpose, so every forward agrees bit for bit."""
    if dtype == torch.float32 and cin > 128:
        pytest.skip("fp32 contraction is limited to 128 channels")
    print(f"pretransposed seed={seed} cin={cin} cout={cout} k={k} {dtype}", flush=True)
    c, t = _subm_case(seed, 12, 0.35, 2, k, cin, cout, dtype)
    x, w, b = cuda(t["feats"]), cuda(t["weight"]), cuda(t["bias"])
    assert torch.equal(spc.transpose_weight(w), w.transpose(1, 2).contiguous())
    km = spc.build_kmap(cuda(c), 2, (12,) * 3, k, orders=True)
    nbr, order = (km["nbr"], km["order"]) if k > 1 else (None, None)
    n = c.shape[0]
    direct = spc.subm_conv_fwd(x, w, b, nbr, order, pretranspose=False)
    assert torch.equal(direct, spc.subm_conv_fwd(x, w, b, nbr, order, pretranspose=True))
    res = cuda(t["grad"][:, :cout]) if t["grad"].shape[1] >= cout else None
    f0 = spc.conv_fwd_fused(x, w, b, nbr, n, order, residual=res, relu=True, pretranspose=False)
    assert torch.equal(f0, spc.conv_fwd_fused(x, w, b, nbr, n, order, residual=res, relu=True, pretranspose=True))
    if k > 1:  # a strided layer and its inverse on the same sites
        ks = spc.build_kmap(cuda(c), 2, (12,) * 3, 3, 2, 1, 1, subm=False, orders=True)
        s0 = spc.sparse_conv_fwd(x, w, b, ks["nbr"], ks["n_out"], ks["order"], pretranspose=False)
        assert torch.equal(s0, spc.sparse_conv_fwd(x, w, b, ks["nbr"], ks["n_out"], ks["order"], pretranspose=True))
        ref = O.strided_kmap(c, 2, (12,) * 3, 3, 2, 1, 1)
        assert_close(s0, OC.conv_fwd(t["feats"], t["weight"], t["bias"], ref["nbr_out"]), TOL[dtype], "strided")
        wi = w.transpose(1, 2).contiguous()  # cout -> cin back onto the input sites
        i0 = spc.sparse_inverse_conv_fwd(s0, wi, None, ks["nbr_in"], n, ks["order_in"], pretranspose=False)
        assert torch.equal(i0, spc.sparse_inverse_conv_fwd(s0, wi, None, ks["nbr_in"], n, ks["order_in"],
                                                            pretranspose=True))


def test_deterministic():
    c, t = _subm_case(8, 20, 0.3, 2, 3, 64, 64, torch.bfloat16)
    km = spc.build_kmap(cuda(c), 2, (20,) * 3, 3, orders=True)
    x, w, g = cuda(t["feats"]), cuda(t["weight"]), cuda(t["grad"])
    o1, o2 = spc.subm_conv_fwd(x, w, None, km["nbr"]), spc.subm_conv_fwd(x, w, None, km["nbr"])
    assert torch.equal(o1, o2)
    # the processing order regroups rows into tiles but never changes a result
    assert torch.equal(o1, spc.subm_conv_fwd(x, w, None, km["nbr"], km["order"]))
    d1 = spc.conv_bwd_input(g, w, km["nbr"], True, c.shape[0])
    assert torch.equal(d1, spc.conv_bwd_input(g, w, km["nbr"], True, c.shape[0], km["order"]))
    a = spc.conv_bwd_filter(x, g, 27, km["pair_ptr"], km["pair_in"], km["pair_out"], True)
    b = spc.conv_bwd_filter(x, g, 27, km["pair_ptr"], km["pair_in"], km["pair_out"], True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ---------------------------------------------------------------- full-size workloads

def test_workload_uniform32_fp32():
    w = W.workload("subm_k3_f32_uniform32", with_grad=True)
    t = {"feats": w.feats, "weight": w.weight, "bias": w.bias, "grad": w.grad}
    run_subm_layer(w.coords, w.batch, w.shape, 3, t, w.dtype, what=w.name)


def test_workload_lidar_fp16():
    w = W.workload("subm_k3_f16_lidar120k", with_grad=True)
    t = {"feats": w.feats, "weight": w.weight, "bias": None, "grad": w.grad}
    run_subm_layer(w.coords, w.batch, w.shape, 3, t, w.dtype, what=w.name)


def test_workload_shells_bf16_k3_then_k1():
    w = W.workload("subm_k3_k1_bf16_shells128")
    print(f"{w.name} n={w.n}", flush=True)
    km = spc.build_kmap(cuda(w.coords), w.batch, w.shape, 3, pairs=False, orders=True)
    nbr_ref = O.subm_kmap(w.coords, w.shape, 3)
    x, wt, w1 = cuda(w.feats), cuda(w.weight), cuda(w.extra["weight_k1"])
    y = spc.subm_conv_fwd(x, wt, None, km["nbr"], km["order"])
    y_ref = OC.conv_fwd(w.feats, w.weight, None, nbr_ref)
    assert_close(y, y_ref, TOL[w.dtype], "k3")
    # layer 2 (k=1) consumes the GPU's own bf16 layer-1 output; the oracle gets the same values
    z = spc.subm_conv_fwd(y, w1, None, None)
    assert_close(z, OC.conv_fwd(y.cpu(), w.extra["weight_k1"], None, np.arange(w.n)[None]), TOL[w.dtype], "k1")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n,cin,cout", [
    (300_001, 32, 64),   # 2,344 tiles: several per workgroup, ragged last tile
    (70_000, 128, 128),  # full 128-channel tiles
    (1_000, 64, 16),     # fewer tiles than workgroups
])
def test_k1_layer_over_many_tiles(dtype, n, cin, cout):
    """The identity map of a k = 1 layer, whose workgroups each walk several
    tiles with the weight slab staged once: forward (both weight layouts) and
    dinput against the oracle."""
    t = W.small_layer(170 + cin, np.zeros((n, 4), np.int32), cin, cout, 1, dtype)
    ident = np.arange(n)[None]
    x, w, b, g = cuda(t["feats"]), cuda(t["weight"]), cuda(t["bias"]), cuda(t["grad"])
    print(f"k1 walk n={n} {cin}->{cout} {dtype}", flush=True)
    out = spc.subm_conv_fwd(x, w, b, None)
    assert_close(out, OC.conv_fwd(t["feats"], t["weight"], t["bias"], ident), TOL[dtype], "k1 fwd")
    for pre in (False, True):
        assert torch.equal(spc.subm_conv_fwd(x, w, b, None, pretranspose=pre), out), f"pretranspose={pre}"
    din = spc.conv_bwd_input(g, w, None, True, n)
    assert_close(din, OC.conv_bwd_input(t["grad"], t["weight"], ident, n), TOL[dtype], "k1 dinput")
    assert torch.equal(spc.conv_bwd_input(g, w, None, True, n), din)  # run twice: identical


def test_workload_strided_lidar_fp16():
    w = W.workload("strided_k3s2_f16_lidar120k")
    km = spc.build_kmap(cuda(w.coords), w.batch, w.shape, 3, 2, 1, 1, subm=False, orders=True)
    ref = O.strided_kmap(w.coords, w.batch, w.shape, 3, 2, 1, 1)
    M = km["n_out"]
    print(f"{w.name} n={w.n} M={M}", flush=True)
    g = W.grad_for(w.extra["grad_rng"], M, w.cout, w.dtype)
    x, wt, gd = cuda(w.feats), cuda(w.weight), cuda(g)
    out = spc.sparse_conv_fwd(x, wt, None, km["nbr"], M, km["order"])
    assert_close(out, OC.conv_fwd(w.feats, w.weight, None, ref["nbr_out"]), TOL[w.dtype], "fwd")
    din = spc.conv_bwd_input(gd, wt, km["nbr_in"], False, w.n, km["order_in"])
    assert_close(din, OC.conv_bwd_input(g, w.weight, ref["nbr_out"], w.n), TOL[w.dtype], "din")
    dw, _ = spc.conv_bwd_filter(x, gd, 27, km["pair_ptr"], km["pair_in"], km["pair_out"])
    dw_ref = OC.conv_bwd_filter(w.feats, g, ref["nbr_out"])
    assert_close(dw, dw_ref, TOL_DW, "dw")
    hygon_check(out, OC.conv_fwd(w.feats, w.weight, None, ref["nbr_out"]), 64, 128, False, "fwd")
    hygon_check(dw, dw_ref, 64, 128, False, "dw")


def test_workload_train_shells_bf16():
    w = W.workload("train_subm_k3_bf16_shells96")
    t = {"feats": w.feats, "weight": w.weight, "bias": None, "grad": w.grad}
    errs = run_subm_layer(w.coords, w.batch, w.shape, 3, t, w.dtype, what=w.name)
    print("errors", errs, flush=True)


@pytest.mark.parametrize("dtype,cin,cout", [(torch.float16, 64, 48), (torch.float32, 32, 16)])
def test_many_tiles_with_empty_tiles(dtype, cin, cout):
    # more 128-row tiles than workgroups resident at once, whole tiles whose
    # rows hit no offset, and a ragged tail: a grid that walks several tiles
    # per workgroup must give every row its own sum and leave empty rows at
    # the bias
    r = W.rng(77)
    n_src, M, K = 5000, 140_037, 27
    nbr = np.where(r.random((K, M)) < 0.15, r.integers(0, n_src, (K, M)), -1).astype(np.int32)
    tiles = (M + 127) // 128
    for j in np.nonzero(r.random(tiles) < 0.3)[0]:
        nbr[:, j * 128:(j + 1) * 128] = -1
    t = W.small_layer(78, np.zeros((n_src, 4), np.int32), cin, cout, K, dtype)
    print(f"synthetic map M={M} n_src={n_src} {dtype} {cin}->{cout}", flush=True)
    x, w, b = cuda(t["feats"]), cuda(t["weight"]), cuda(t["bias"])
    nbr_mk = cuda(np.ascontiguousarray(nbr.T))
    out = spc.sparse_conv_fwd(x, w, b, nbr_mk, M)
    assert_close(out, OC.conv_fwd(t["feats"], t["weight"], t["bias"], nbr), TOL[dtype], "fwd")
    perm = cuda(r.permutation(M).astype(np.int32))
    assert torch.equal(out, spc.sparse_conv_fwd(x, w, b, nbr_mk, M, perm))


# ------------------------------------------------ inverse (upsampling) conv

def run_inverse(c, batch, shape, k, s, p, d, t, dtype, ref, what=""):
    """Inverse forward on a strided map, and its dinput / dfilter / dbias through
    the existing backward calls (map and pair lists exchanged), vs the oracle."""
    km = spc.build_kmap(cuda(c), batch, shape, k, s, p, d, subm=False, orders=True)
    M, N = km["n_out"], c.shape[0]
    print(f"inverse conv {what} N={N} M={M} k={k} s={s} {tuple(t['weight'].shape)} {dtype}", flush=True)
    x, w, g = cuda(t["feats"]), cuda(t["weight"]), cuda(t["grad"])
    b = cuda(t["bias"]) if t.get("bias") is not None else None
    out = spc.sparse_inverse_conv_fwd(x, w, b, km["nbr_in"], N, km["order_in"])
    assert_close(out, OC.inverse_conv_fwd(t["feats"], t["weight"], t["bias"], ref["nbr_out"], N), TOL[dtype], "fwd")
    assert torch.equal(out, spc.sparse_inverse_conv_fwd(x, w, b, km["nbr_in"], N))  # order never changes a result
    din = spc.conv_bwd_input(g, w, km["nbr"], False, M, km["order"])
    assert_close(din, OC.inverse_conv_bwd_input(t["grad"], t["weight"], ref["nbr_out"], M), TOL[dtype], "din")
    dw, db = spc.conv_bwd_filter(x, g, k ** 3, km["pair_ptr"], km["pair_out"], km["pair_in"], want_dbias=True)
    assert_close(dw, OC.inverse_conv_bwd_filter(t["feats"], t["grad"], ref["nbr_out"]), TOL_DW, "dw")
    assert_close(db, OC.conv_bwd_bias(t["grad"]), TOL_DW, "dbias")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape,k,s,p,d,cin,cout", [
    ((12, 14, 10), 3, 2, 1, 1, 32, 16), ((15, 13, 11), 2, 2, 0, 1, 16, 48), ((11, 11, 11), 3, 1, 0, 2, 64, 32),
])
def test_inverse_small(dtype, shape, k, s, p, d, cin, cout):
    c = W.tiny_grid(W.rng(45 + k + s), min(shape), 0.25, 2)
    ref = O.strided_kmap(c, 2, shape, k, s, p, d)
    # coarse features [M, cin], the inverse layer's weight [K, cin, cout], a fine gradient [N, cout]
    t = W.small_layer(56, ref["out_coords"], cin, cout, k ** 3, dtype, n_out=c.shape[0])
    run_inverse(c, 2, shape, k, s, p, d, t, dtype, ref)


def test_workload_inverse_lidar_fp16():
    # the upsampling back from the strided lidar layer: 128 coarse channels -> 64
    w = W.workload("strided_k3s2_f16_lidar120k")
    ref = O.strided_kmap(w.coords, w.batch, w.shape, 3, 2, 1, 1)
    t = W.small_layer(57, ref["out_coords"], 128, 64, 27, w.dtype, bias=False, n_out=w.n)
    run_inverse(w.coords, w.batch, w.shape, 3, 2, 1, 1, t, w.dtype, ref, what=w.name)


# ------------------------------------------------ fused conv-add-relu epilogue

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("kind", ["subm", "strided", "inverse", "k1"])
def test_fused_epilogue(dtype, kind):
    shape = (12, 14, 10)
    c = W.tiny_grid(W.rng(160), min(shape), 0.3, 2)
    cin, cout = 32, 48
    if kind in ("subm", "k1"):
        k = 3 if kind == "subm" else 1
        km = spc.build_kmap(cuda(c), 2, shape, k, orders=True) if k > 1 else None
        nbr = O.subm_kmap(c, shape, k) if k > 1 else np.arange(c.shape[0])[None]
        src_n, rows = c.shape[0], c.shape[0]
        m, order = (km["nbr"], km["order"]) if k > 1 else (None, None)
    else:
        k = 3
        km = spc.build_kmap(cuda(c), 2, shape, 3, 2, 1, 1, subm=False, orders=True)
        ref = O.strided_kmap(c, 2, shape, 3, 2, 1, 1)
        M = ref["out_coords"].shape[0]
        if kind == "strided":
            nbr, src_n, rows, m, order = ref["nbr_out"], c.shape[0], M, km["nbr"], km["order"]
        else:
            nbr, src_n, rows, m, order = ref["nbr_in"], M, c.shape[0], km["nbr_in"], km["order_in"]
    t = W.small_layer(161, np.zeros((src_n, 4), np.int32), cin, cout, k ** 3, dtype)
    res = W.small_layer(162, np.zeros((rows, 4), np.int32), cout, cout, 1, dtype)["feats"]
    x, w, b, r = cuda(t["feats"]), cuda(t["weight"]), cuda(t["bias"]), cuda(res)
    print(f"fused {kind} rows={rows} src={src_n} {dtype}", flush=True)
    for relu in (False, True):
        out = spc.conv_fwd_fused(x, w, b, m, rows, order, residual=r, relu=relu)
        assert_close(out, OC.conv_fwd_fused(t["feats"], t["weight"], t["bias"], nbr, res, relu), TOL[dtype],
                     f"fused relu={relu}")
        if relu:
            assert (out.float() >= 0).all()
    # without residual and activation it is the plain forward, bit for bit
    plain = spc.conv_fwd_fused(x, w, b, m, rows, order)
    if kind in ("subm", "k1"):
        assert torch.equal(plain, spc.subm_conv_fwd(x, w, b, m, order))
    elif kind == "strided":
        assert torch.equal(plain, spc.sparse_conv_fwd(x, w, b, m, rows, order))
    else:
        assert torch.equal(plain, spc.sparse_inverse_conv_fwd(x, w, b, m, rows, order))
    # in place: the residual buffer is also the output
    buf = r.clone()
    spc.conv_fwd_fused(x, w, b, m, rows, order, residual=buf, relu=True, out=buf)
    assert torch.equal(buf, spc.conv_fwd_fused(x, w, b, m, rows, order, residual=r, relu=True))


def test_workload_fused_lidar_fp16():
    # the submanifold lidar layer as a residual block: relu(conv(x) + x)
    w = W.workload("subm_k3_f16_lidar120k")
    km = spc.build_kmap(cuda(w.coords), w.batch, w.shape, 3, orders=True)
    nbr_ref = O.subm_kmap(w.coords, w.shape, 3)
    x, wt = cuda(w.feats), cuda(w.weight)
    print(f"{w.name} fused n={w.n}", flush=True)
    out = spc.conv_fwd_fused(x, wt, None, km["nbr"], w.n, km["order"], residual=x, relu=True)
    assert_close(out, OC.conv_fwd_fused(w.feats, w.weight, None, nbr_ref, w.feats, True), TOL[w.dtype], "fused")


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("case", ["ragged", "full_block", "sparse", "unordered"])
def test_subm_128_channel_layers(dtype, case):
    """128 -> 128 submanifold layers (the shell workload's shape, with weights
    pre-transposed by the binding): forward, fused residual + ReLU and dinput
    against the oracle, over several tiles with a ragged tail, a full block
    (every tile hits all 27 offsets), a sparse grid (tiles of one or two
    offsets) and rows in natural order; the forward also bit for bit against
    the per-tile-transpose staging."""
    r = W.rng(700 + len(case))
    if case == "full_block":
        c, side, batch = W.random_block(r, 12), 12, 1
    elif case == "sparse":
        c, side, batch = W.uniform_grid(r, 700, 40, 2), 40, 2
    else:
        c, side, batch = W.tiny_grid(r, 14, 0.4, 2), 14, 2
    print(f"subm 128 channels {case} n={c.shape[0]} {dtype}", flush=True)
    t = W.small_layer(700 + len(case), c, 128, 128, 27, dtype)
    km = spc.build_kmap(cuda(c), batch, (side,) * 3, 3, orders=case != "unordered")
    nbr = O.subm_kmap(c, (side,) * 3, 3)
    order = km.get("order")
    x, w, b, g = cuda(t["feats"]), cuda(t["weight"]), cuda(t["bias"]), cuda(t["grad"])
    out = spc.subm_conv_fwd(x, w, b, km["nbr"], order)
    assert_close(out, OC.conv_fwd(t["feats"], t["weight"], t["bias"], nbr), TOL[dtype], "fwd")
    assert torch.equal(out, spc.subm_conv_fwd(x, w, b, km["nbr"], order, pretranspose=False))
    res = cuda(t["grad"])
    fused = spc.conv_fwd_fused(x, w, b, km["nbr"], c.shape[0], order, residual=res, relu=True)
    assert_close(fused, OC.conv_fwd_fused(t["feats"], t["weight"], t["bias"], nbr, t["grad"], True), TOL[dtype],
                 "fused")
    din = spc.conv_bwd_input(g, w, km["nbr"], True, c.shape[0], order)
    assert_close(din, OC.conv_bwd_input(t["grad"], t["weight"], nbr, c.shape[0]), TOL[dtype], "din")


@pytest.mark.parametrize("dtype,cin,cout", [(torch.float16, 64, 128), (torch.bfloat16, 128, 64),
                                            (torch.float32, 32, 48)])
def test_dev_rows_forward_equals_the_host_rows_forward(dtype, cin, cout):
    # the strided forward over a map that left its count on the device
    # (grid sized by the capacity, rows past M untouched) gives the host-row
    # forward's rows bit for bit, in both weight layouts and with the fused
    # residual + ReLU epilogue; the host-row forward is checked against the
    # oracle by the strided workload tests
    w = W.workload("strided_k3s2_f16_lidar120k")
    c = cuda(w.coords)
    cap = spc.strided_out_bound(w.n, w.batch, w.shape, 3, 2, 1, 1)
    km = spc.build_kmap(c, w.batch, w.shape, 3, 2, 1, 1, subm=False, orders=True)
    ka = spc.build_kmap(c, w.batch, w.shape, 3, 2, 1, 1, subm=False, orders=True, out_cap=cap, device_count=True)
    M = km["n_out"]
    assert int(ka["n_out_dev"].item()) == M
    t = W.small_layer(310 + cin, w.coords, cin, cout, 27, dtype)
    x, wt = cuda(t["feats"]), cuda(t["weight"])
    bias = cuda(t["bias"]) if t["bias"] is not None else None
    res = cuda(W.grad_for(W.rng(311), cap, cout, dtype))
    wT = spc.transpose_weight(wt)
    sentinel = torch.full((cap, cout), 3.0, dtype=dtype, device=x.device)
    print(f"dev-rows forward {dtype} {cin}->{cout} M={M} cap={cap}", flush=True)
    ref = spc.sparse_conv_fwd(x, wt, bias, km["nbr"], M, km["order"], pretranspose=False)
    ref_t = spc.conv_fwd_wt(x, wT, bias, km["nbr"], M, False, km["order"])
    ref_f = spc.conv_fwd_fused(x, wt, bias, km["nbr"], M, km["order"], residual=res[:M].contiguous(), relu=True,
                               pretranspose=False)
    for weight_t, wgt, want, kw in ((False, wt, ref, {}), (True, wT, ref_t, {}),
                                    (False, wt, ref_f, {"residual": res, "relu": True})):
        out = sentinel.clone()
        spc.conv_fwd_dev_rows(x, wgt, bias, ka["nbr"], ka["n_out_dev"], cap, ka["order"], weight_t=weight_t,
                              out=out, **kw)
        assert torch.equal(out[:M], want), (weight_t, kw)
        assert torch.equal(out[M:], sentinel[M:]), "rows past the count were written"
    # a count above the capacity (an overflowed map) writes nothing
    over = torch.full((4,), cap + 1, dtype=torch.int32, device=x.device)
    out = sentinel.clone()
    spc.conv_fwd_dev_rows(x, wt, bias, ka["nbr"], over[:1], cap, ka["order"], out=out)
    assert torch.equal(out, sentinel)
