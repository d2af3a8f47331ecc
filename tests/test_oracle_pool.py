"""Pins of the oracle's sparse max pooling: torch's dense max_pool3d and its
autograd on grids whose empty sites hold -inf (float64, CPU), and a
hand-built tie."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workloads as W
from oracle import kmap as O
from oracle import pool as P
from tests.dense import densify, sample

GEOMS = [((7, 8, 6), 2, 2, 0, 1), ((8, 7, 9), 3, 2, 1, 1), ((6, 7, 8), 3, 1, 1, 1), ((9, 8, 7), 3, 2, 0, 2)]


def _case(shape, k, s, p, d, seed, C=5):
    c = W.tiny_grid(W.rng(seed), min(shape), 0.3, 2)
    res = O.strided_kmap(c, 2, shape, k, s, p, d)
    x = W.rng(seed, "feats").standard_normal((c.shape[0], C))
    return c, res, x


@pytest.mark.parametrize("shape,k,s,p,d", GEOMS)
def test_maxpool_equals_dense_max_pool3d(shape, k, s, p, d):
    c, res, x = _case(shape, k, s, p, d, 170 + k + s + d)
    out, argk = P.maxpool_fwd(x, res["nbr_out"])
    dense = F.max_pool3d(densify(c, x, 2, shape, fill=-np.inf), k, s, p, dilation=d)
    np.testing.assert_array_equal(out, sample(dense, res["out_coords"]).numpy())
    assert (argk != P.NO_ARG).all()  # every strided output has an input


@pytest.mark.parametrize("shape,k,s,p,d", GEOMS)
def test_maxpool_backward_equals_autograd(shape, k, s, p, d):
    c, res, x = _case(shape, k, s, p, d, 180 + k + s + d)
    xd = densify(c, x, 2, shape, fill=-np.inf).requires_grad_(True)
    y = F.max_pool3d(xd, k, s, p, dilation=d)
    g = W.rng(181, "grad").standard_normal((res["out_coords"].shape[0], x.shape[1]))
    gd = torch.zeros_like(y)
    oc = torch.as_tensor(res["out_coords"].astype(np.int64))
    gd[oc[:, 0], :, oc[:, 1], oc[:, 2], oc[:, 3]] = torch.as_tensor(g)
    (y * gd).sum().backward()
    _, argk = P.maxpool_fwd(x, res["nbr_out"])
    np.testing.assert_allclose(P.maxpool_bwd(g, argk, res["nbr_out"], c.shape[0]), sample(xd.grad, c).numpy(),
                               rtol=1e-13, atol=1e-13)


def test_maxpool_tie_goes_to_first_offset():
    # a 2x2x2 pool over two voxels with equal values in channel 0: the one at
    # the smaller offset wins, and only it receives the gradient
    c = np.array([[0, 1, 1, 1], [0, 0, 0, 0]], np.int32)  # offsets 7 and 0 of output (0,0,0)
    res = O.strided_kmap(c, 1, (2, 2, 2), 2, 2, 0, 1)
    x = np.array([[3.0, 1.0], [3.0, 2.0]])
    out, argk = P.maxpool_fwd(x, res["nbr_out"])
    np.testing.assert_array_equal(out, [[3.0, 2.0]])
    np.testing.assert_array_equal(argk, [[0, 0]])
    din = P.maxpool_bwd(np.array([[10.0, 20.0]]), argk, res["nbr_out"], 2)
    np.testing.assert_array_equal(din, [[0.0, 0.0], [10.0, 20.0]])


def test_maxpool_negative_values_and_lone_input():
    # a window with one input passes it through unchanged, however negative
    c = np.array([[0, 0, 0, 0]], np.int32)
    res = O.strided_kmap(c, 1, (2, 2, 2), 2, 2, 0, 1)
    out, argk = P.maxpool_fwd(np.array([[-7.5, -0.25]]), res["nbr_out"])
    np.testing.assert_array_equal(out, [[-7.5, -0.25]])
    np.testing.assert_array_equal(argk, [[0, 0]])
