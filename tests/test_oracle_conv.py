"""Pins of the oracle's convolution arithmetic against torch's dense conv3d and
its autograd (float64 on the CPU), closed forms and the adjoint identity.
A few tests plant a plausible mistake in the oracle and check a pin catches it."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import conv as C
from oracle import kmap as O
from tests.dense import dense_conv, dense_conv_transpose, densify, sample, torch_weight


def _layer(seed, c, cin, cout, K, dtype=torch.float64, n_out=None):
    t = W.small_layer(seed, c, cin, cout, K, torch.float32, n_out=n_out)
    return {k: (v.to(dtype) if isinstance(v, torch.Tensor) else v) for k, v in t.items()}


@pytest.mark.parametrize("seed,side,fill,batch,k,cin,cout", [
    (1, 6, 0.3, 1, 3, 4, 5), (2, 7, 0.1, 2, 3, 3, 2), (3, 5, 0.5, 1, 5, 2, 3),
    (4, 6, 0.25, 2, 1, 4, 4), (5, 9, 0.15, 1, 3, 8, 8),
])
def test_subm_fwd_equals_dense_conv3d(seed, side, fill, batch, k, cin, cout):
    c = W.tiny_grid(W.rng(seed), side, fill, batch)
    t = _layer(seed, c, cin, cout, k ** 3)
    nbr = O.subm_kmap(c, (side,) * 3, k)
    got = C.conv_fwd(t["feats"], t["weight"], t["bias"], nbr)
    ref = sample(dense_conv(c, t["feats"], t["weight"], t["bias"], batch, (side,) * 3, k), c)
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("shape,k,s,p,d", [
    ((7, 8, 6), 3, 2, 1, 1), ((8, 8, 8), 2, 2, 0, 1), ((9, 7, 8), 3, 1, 0, 2), ((8, 9, 7), 3, 3, 2, 1),
])
def test_strided_fwd_equals_dense_conv3d(shape, k, s, p, d):
    c = W.tiny_grid(W.rng(60 + s + k), min(shape), 0.2, 2)
    res = O.strided_kmap(c, 2, shape, k, s, p, d)
    t = _layer(7, c, 3, 4, k ** 3)
    got = C.conv_fwd(t["feats"], t["weight"], t["bias"], res["nbr_out"])
    dense = dense_conv(c, t["feats"], t["weight"], t["bias"], 2, shape, k, s, p, d)
    ref = sample(dense, res["out_coords"])
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_single_voxel_is_centre_tap():
    c = np.array([[0, 2, 3, 4]], np.int32)
    t = _layer(8, c, 6, 5, 27)
    nbr = O.subm_kmap(c, (8, 8, 8), 3)
    got = C.conv_fwd(t["feats"], t["weight"], t["bias"], nbr)
    want = t["bias"].numpy() + t["feats"].numpy()[0] @ t["weight"].numpy()[13]
    np.testing.assert_allclose(got[0], want, rtol=1e-14)


def test_full_block_equals_dense_everywhere():
    c = W.random_block(W.rng(9), 4, origin=(1, 1, 1))
    t = _layer(9, c, 3, 3, 27)
    got = C.conv_fwd(t["feats"], t["weight"], None, O.subm_kmap(c, (6, 6, 6), 3))
    dense = dense_conv(c, t["feats"], t["weight"], None, 1, (6, 6, 6), 3)
    np.testing.assert_allclose(got, sample(dense, c).numpy(), rtol=1e-12, atol=1e-12)


def test_linearity():
    c = W.tiny_grid(W.rng(10), 6, 0.3, 1)
    nbr = O.subm_kmap(c, (6, 6, 6), 3)
    a, b = _layer(10, c, 4, 4, 27), _layer(11, c, 4, 4, 27)
    f = lambda x, w: C.conv_fwd(x, w, None, nbr)
    np.testing.assert_allclose(f(a["feats"] * 2 + b["feats"], a["weight"]),
                               2 * f(a["feats"], a["weight"]) + f(b["feats"], a["weight"]), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(f(a["feats"], a["weight"] - 3 * b["weight"]),
                               f(a["feats"], a["weight"]) - 3 * f(a["feats"], b["weight"]), rtol=1e-12, atol=1e-12)


def _autograd(c, t, batch, shape, k, s, p, d, out_coords):
    x = densify(c, t["feats"], batch, shape).requires_grad_(True)
    w = torch_weight(t["weight"], k).requires_grad_(True)
    bias = t["bias"].clone().requires_grad_(True)
    y = torch.nn.functional.conv3d(x, w, bias, stride=s, padding=p, dilation=d)
    g = torch.zeros_like(y)
    oc = torch.as_tensor(out_coords.astype(np.int64))
    g[oc[:, 0], :, oc[:, 1], oc[:, 2], oc[:, 3]] = t["grad"]
    (y * g).sum().backward()
    din = sample(x.grad, c).numpy()
    dw = w.grad.permute(2, 3, 4, 1, 0).reshape(k ** 3, w.shape[1], w.shape[0]).numpy()
    return din, dw, bias.grad.numpy()


@pytest.mark.parametrize("kind", ["subm3", "subm5", "strided", "strided_dil"])
def test_backward_equals_autograd(kind):
    shape = (7, 8, 6)
    c = W.tiny_grid(W.rng(70), 6, 0.3, 2)
    if kind.startswith("subm"):
        k = int(kind[-1])
        s, p, d = 1, k // 2, 1
        nbr, oc = O.subm_kmap(c, shape, k), c
    else:
        k, s, p, d = (3, 2, 1, 1) if kind == "strided" else (3, 1, 0, 2)
        res = O.strided_kmap(c, 2, shape, k, s, p, d)
        nbr, oc = res["nbr_out"], res["out_coords"]
    t = _layer(71, c, 3, 5, k ** 3, n_out=oc.shape[0])
    din, dw, db = _autograd(c, t, 2, shape, k, s, p, d, oc)
    np.testing.assert_allclose(C.conv_bwd_input(t["grad"], t["weight"], nbr, c.shape[0]), din,
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(C.conv_bwd_filter(t["feats"], t["grad"], nbr), dw, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(C.conv_bwd_bias(t["grad"]), db, rtol=1e-12, atol=1e-12)


def test_adjoint_identity():
    c = W.tiny_grid(W.rng(80), 9, 0.2, 2)
    res = O.strided_kmap(c, 2, (9, 9, 9), 3, 2, 1, 1)
    t = _layer(81, c, 6, 7, 27, n_out=res["out_coords"].shape[0])
    x, w, g = t["feats"].numpy(), t["weight"].numpy(), t["grad"].numpy()
    y = C.conv_fwd(x, w, None, res["nbr_out"])
    lhs = (y * g).sum()
    assert np.isclose(lhs, (x * C.conv_bwd_input(g, w, res["nbr_out"], x.shape[0])).sum(), rtol=1e-12)
    assert np.isclose(lhs, (w * C.conv_bwd_filter(x, g, res["nbr_out"])).sum(), rtol=1e-12)


def test_rows_variant_matches_full():
    c = W.tiny_grid(W.rng(90), 7, 0.3, 1)
    t = _layer(90, c, 4, 3, 27)
    nbr = O.subm_kmap(c, (7, 7, 7), 3)
    rows = [0, 3, c.shape[0] - 1]
    np.testing.assert_allclose(C.conv_fwd_rows(t["feats"], t["weight"], t["bias"], nbr, rows),
                               C.conv_fwd(t["feats"], t["weight"], t["bias"], nbr)[rows], rtol=1e-13)


# ------------------------------------------------- planted mistakes (CPU only)

def _dense_pin_holds(monkeypatch_fn=None):
    c = W.tiny_grid(W.rng(100), 6, 0.35, 1)
    t = _layer(100, c, 4, 4, 27)
    nbr = O.subm_kmap(c, (6, 6, 6), 3)
    got = C.conv_fwd(t["feats"], t["weight"], t["bias"], nbr)
    ref = sample(dense_conv(c, t["feats"], t["weight"], t["bias"], 1, (6, 6, 6), 3), c).numpy()
    return np.allclose(got, ref, rtol=1e-10, atol=1e-10)


def test_planted_offset_sign_flip_is_caught(monkeypatch):
    real = O.subm_offsets
    monkeypatch.setattr(O, "subm_offsets", lambda k: -real(k))
    assert not _dense_pin_holds()


def test_planted_transposed_weight_is_caught(monkeypatch):
    real = C.f64
    calls = {"n": 0}

    def f64(t):
        a = real(t)
        calls["n"] += 1
        return a.transpose(0, 2, 1).copy() if a.ndim == 3 else a
    monkeypatch.setattr(C, "f64", f64)
    assert not _dense_pin_holds()


def test_planted_dropped_offset_is_caught(monkeypatch):
    real = O.subm_kmap

    def dropped(*a, **kw):
        nbr = real(*a, **kw)
        nbr[-1] = -1
        return nbr
    monkeypatch.setattr(O, "subm_kmap", dropped)
    assert not _dense_pin_holds()


# ------------------------------------------------ inverse (upsampling) conv

def _inverse_case(shape, k, s, p, d, seed, cin=3, cout=4):
    c = W.tiny_grid(W.rng(seed), min(shape), 0.25, 2)
    res = O.strided_kmap(c, 2, shape, k, s, p, d)
    M = res["out_coords"].shape[0]
    # the coarse layer's features, the inverse layer's weight [K, Cin, Cout], and a
    # gradient on the fine sites
    t = _layer(seed + 1, res["out_coords"], cin, cout, k ** 3, n_out=c.shape[0])
    return c, res, M, t


@pytest.mark.parametrize("shape,k,s,p,d", [
    ((7, 8, 6), 3, 2, 1, 1), ((8, 8, 7), 2, 2, 0, 1), ((9, 7, 8), 3, 1, 0, 2), ((8, 9, 7), 3, 3, 2, 1),
])
def test_inverse_fwd_equals_dense_conv_transpose3d(shape, k, s, p, d):
    c, res, M, t = _inverse_case(shape, k, s, p, d, 110 + k + s)
    got = C.inverse_conv_fwd(t["feats"], t["weight"], t["bias"], res["nbr_out"], c.shape[0])
    oshape = O.out_shape(shape, k, s, p, d)
    dense = dense_conv_transpose(res["out_coords"], t["feats"], t["weight"], t["bias"], 2, oshape, shape, k, s, p, d)
    np.testing.assert_allclose(got, sample(dense, c).numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("shape,k,s,p,d", [((7, 8, 6), 3, 2, 1, 1), ((8, 8, 7), 2, 2, 0, 1)])
def test_inverse_backward_equals_autograd(shape, k, s, p, d):
    c, res, M, t = _inverse_case(shape, k, s, p, d, 120 + k)
    oshape = O.out_shape(shape, k, s, p, d)
    x = densify(res["out_coords"], t["feats"], 2, oshape).requires_grad_(True)
    w = torch.as_tensor(t["weight"].numpy(), dtype=torch.float64).requires_grad_(True)
    wt = w.reshape(k, k, k, w.shape[1], w.shape[2]).permute(3, 4, 0, 1, 2)
    op = tuple(f - ((q - 1) * s - 2 * p + d * (k - 1) + 1) for f, q in zip(shape, oshape))
    y = torch.nn.functional.conv_transpose3d(x, wt, None, stride=s, padding=p, output_padding=op, dilation=d)
    g = torch.zeros_like(y)
    cc = torch.as_tensor(c.astype(np.int64))
    g[cc[:, 0], :, cc[:, 1], cc[:, 2], cc[:, 3]] = torch.as_tensor(t["grad"].numpy(), dtype=torch.float64)
    (y * g).sum().backward()
    np.testing.assert_allclose(C.inverse_conv_bwd_input(t["grad"], t["weight"], res["nbr_out"], M),
                               sample(x.grad, res["out_coords"]).numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(C.inverse_conv_bwd_filter(t["feats"], t["grad"], res["nbr_out"]), w.grad.numpy(),
                               rtol=1e-12, atol=1e-12)


def test_inverse_is_adjoint_of_strided_conv():
    # <inverse(x; W), z> = <x, strided conv(z; W^T)> on the same saved map
    c, res, M, t = _inverse_case((9, 9, 9), 3, 2, 1, 1, 130, cin=5, cout=6)
    x, w, z = t["feats"].numpy(), t["weight"].numpy(), t["grad"].numpy()
    lhs = (C.inverse_conv_fwd(x, w, None, res["nbr_out"], c.shape[0]) * z).sum()
    rhs = (x * C.conv_fwd(z, w.transpose(0, 2, 1), None, res["nbr_out"])).sum()
    assert np.isclose(lhs, rhs, rtol=1e-12)


def test_planted_inverse_offset_reversal_is_caught(monkeypatch):
    # using W[K-1-k] (the transpose-conv flip that the inverse layer does not do)
    c, res, M, t = _inverse_case((7, 8, 6), 3, 2, 1, 1, 140)
    real = C.f64
    monkeypatch.setattr(C, "f64", lambda a: real(a)[::-1].copy() if real(a).ndim == 3 else real(a))
    got = C.inverse_conv_fwd(t["feats"], t["weight"], t["bias"], res["nbr_out"], c.shape[0])
    dense = dense_conv_transpose(res["out_coords"], t["feats"], t["weight"], t["bias"], 2,
                                 O.out_shape((7, 8, 6), 3, 2, 1, 1), (7, 8, 6), 3, 2, 1)
    assert not np.allclose(got, sample(dense, c).numpy(), rtol=1e-10, atol=1e-10)


# ------------------------------------------------ fused conv-add-relu epilogue

def test_fused_single_voxel_by_hand():
    # one voxel: only the centre tap W[13] acts.  x @ W[13] = [-3, -2, -1];
    # + bias = [-2.5, -6, 0]; + residual = [1.5, -5, 5]; ReLU -> [1.5, 0, 5]
    # (ReLU before the add would give [4, 1, 5])
    c = np.array([[0, 1, 1, 1]], np.int32)
    nbr = O.subm_kmap(c, (3, 3, 3), 3)
    w = np.zeros((27, 2, 3))
    w[13] = [[1, 0, -1], [2, 1, 0]]
    x = np.array([[1.0, -2.0]])
    got = C.conv_fwd_fused(x, w, np.array([0.5, -4.0, 1.0]), nbr, np.array([[4.0, 1.0, 5.0]]), relu=True)
    np.testing.assert_array_equal(got, [[1.5, 0.0, 5.0]])
    got = C.conv_fwd_fused(x, w, np.array([0.5, -4.0, 1.0]), nbr, np.array([[4.0, 1.0, 5.0]]), relu=False)
    np.testing.assert_array_equal(got, [[1.5, -5.0, 5.0]])


def test_fused_equals_dense_conv3d_add_relu():
    c = W.tiny_grid(W.rng(150), 7, 0.3, 1)
    t = _layer(150, c, 4, 5, 27)
    r = _layer(151, c, 5, 5, 27)["feats"]  # a residual [N, 5]
    nbr = O.subm_kmap(c, (7, 7, 7), 3)
    dense = dense_conv(c, t["feats"], t["weight"], t["bias"], 1, (7, 7, 7), 3)
    ref = torch.relu(sample(dense, c) + torch.as_tensor(r.numpy(), dtype=torch.float64)).numpy()
    got = C.conv_fwd_fused(t["feats"], t["weight"], t["bias"], nbr, r, relu=True)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------ the parity measure itself
#
# Every floating-point parity assertion goes through max_rel_err: the bound is
# max|got - ref| <= tol * max|ref|.  These cases are computed by hand, and the
# planted variants below (a mean for the max, a missing abs, a signed
# difference, a scale without abs, an elementwise relative error, silent
# broadcasting) each fail at least one of them.

_MRE_CASES = [
    # (got, ref, expected)
    ([1.0, -4.0, 2.0], [1.0, -4.0, 2.0], 0.0),
    ([1.5, -4.0, 2.0], [1.0, -4.0, 2.0], 0.125),              # 0.5 / 4
    ([[1.0, -3.5], [2.0, -0.25]], [[1.0, -4.0], [2.0, 0.0]], 0.125),  # max 0.5, not the mean 0.1875
    ([-8.0, 3.0], [-8.0, 1.0], 0.25),                         # scale is max|ref| = 8, not max(ref) = 1
    ([0.0, 4.0], [0.0, 5.0], 0.2),                            # |4 - 5| / 5: a signed max would give 0
    ([0.0, 1e-3], [0.0, 0.0], 1e-3),                          # all-zero ref: the absolute error
    ([2.0, 2.0, 2.0, 2.0], [1.0, 1.0, 1.0, 100.0], 0.98),     # 98 / 100, not the max elementwise ratio 1
]


def _check_mre(fn):
    for got, ref, want in _MRE_CASES:
        v = fn(np.array(got), np.array(ref))
        if not np.isclose(v, want, rtol=1e-12, atol=0.0):
            return False
    if fn(np.zeros((0, 4)), np.zeros((0, 4))) != 0.0:
        return False
    try:
        fn(np.ones((1, 3)), np.ones((5, 3)))
        return False  # a [1, C] result must not broadcast against [N, C]
    except ValueError:
        pass
    if fn(np.array([1.0, np.nan]), np.array([1.0, 2.0])) != float("inf"):
        return False
    return True


def test_max_rel_err_hand_cases():
    assert _check_mre(C.max_rel_err)
    # both NaN at the same place counts as equal
    assert C.max_rel_err(np.array([np.nan, 1.0]), np.array([np.nan, 2.0])) == 0.5
    # 16-bit tensors are compared on their exact values: bf16 1.0078125 vs 1.0, scale 3
    got = torch.tensor([1.0078125, 3.0], dtype=torch.bfloat16)
    ref = torch.tensor([1.0, 3.0], dtype=torch.bfloat16)
    assert C.max_rel_err(got, ref) == 0.0078125 / 3.0
    # a NaN fails any tolerance
    assert not (C.max_rel_err(np.array([np.nan]), np.array([1.0])) <= 1e-2)


def _planted(kind):
    def fn(got, ref):
        g, r = np.asarray(got, np.float64), np.asarray(ref, np.float64)
        if kind != "broadcast" and g.shape != r.shape:
            raise ValueError("shape")
        if r.size == 0:
            return 0.0
        if kind == "mean":
            err, scale = np.abs(g - r).mean(), np.abs(r).max()
        elif kind == "no_abs":
            err, scale = (g - r).max(), np.abs(r).max()
        elif kind == "scale_no_abs":
            err, scale = np.abs(g - r).max(), r.max()
        elif kind == "elementwise":
            nz = r != 0
            return float((np.abs(g - r)[nz] / np.abs(r)[nz]).max()) if nz.any() else float(np.abs(g - r).max())
        elif kind == "broadcast":
            err, scale = np.abs(g - r).max(), np.abs(r).max()
        elif kind == "nan_blind":
            err, scale = np.nanmax(np.abs(g - r)), np.abs(r).max()
        return float(err / scale) if scale > 0 else float(err)
    return fn


@pytest.mark.parametrize("kind", ["mean", "no_abs", "scale_no_abs", "elementwise", "broadcast", "nan_blind"])
def test_max_rel_err_planted_variants_fail(kind):
    assert not _check_mre(_planted(kind))
