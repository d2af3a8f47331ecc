"""GPU sparse max pooling vs the oracle: the pooled values and winning
offsets bit for bit (a max is a copy of an input value and its winner an
integer decision on exact values), the backward within the dtype tolerance."""

import numpy as np
import pytest
import torch

import sparse_convolution_hash_amd as spc
import workloads as W
from oracle import kmap as O
from oracle import pool as P
from tests.parity import TOL, assert_close, cuda, host

pytestmark = pytest.mark.gpu

DTYPES = [torch.float32, torch.float16, torch.bfloat16]


def exact(t):
    return t.detach().cpu().to(torch.float64).numpy()


def run_pool(c, batch, shape, k, s, p, d, x, dtype, ref, seed, what=""):
    km = spc.build_kmap(cuda(c), batch, shape, k, s, p, d, subm=False)
    M, N = km["n_out"], c.shape[0]
    print(f"maxpool {what} N={N} M={M} k={k} s={s} p={p} d={d} C={x.shape[1]} {dtype}", flush=True)
    out, argk = spc.sparse_maxpool_fwd(cuda(x), km["nbr"], M)
    ro, ra = P.maxpool_fwd(x, ref["nbr_out"])
    assert np.array_equal(exact(out), ro)
    assert np.array_equal(host(argk), ra)
    out2, none = spc.sparse_maxpool_fwd(cuda(x), km["nbr"], M, want_argk=False)
    assert none is None and torch.equal(out, out2)
    g = W.grad_for(W.rng(seed, "grad"), M, x.shape[1], dtype)
    din = spc.sparse_maxpool_bwd(cuda(g), argk, km["nbr_in"], N)
    assert_close(din, P.maxpool_bwd(g, ra, ref["nbr_out"], N), TOL[dtype], "din")
    assert torch.equal(din, spc.sparse_maxpool_bwd(cuda(g), argk, km["nbr_in"], N))  # run-to-run identical


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape,k,s,p,d,C", [
    ((12, 14, 10), 2, 2, 0, 1, 16), ((11, 13, 12), 3, 2, 1, 1, 48), ((10, 10, 10), 3, 1, 1, 1, 32),
    ((13, 11, 12), 3, 2, 0, 2, 64), ((14, 13, 12), 5, 2, 2, 1, 32),
])
def test_maxpool_small(dtype, shape, k, s, p, d, C):
    c = W.tiny_grid(W.rng(190 + k + s + d), min(shape), 0.3, 2)
    ref = O.strided_kmap(c, 2, shape, k, s, p, d)
    x = W.small_layer(191, c, C, 16, 1, dtype)["feats"]
    run_pool(c, 2, shape, k, s, p, d, x, dtype, ref, 192)


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_maxpool_ties_in_low_precision(dtype):
    # few distinct values, so most windows hold ties: the winner must still be
    # the first offset reaching the maximum
    c = W.tiny_grid(W.rng(193), 12, 0.5, 1)
    ref = O.strided_kmap(c, 1, (12, 12, 12), 3, 2, 1, 1)
    x = torch.from_numpy(W.rng(194, "feats").integers(-3, 4, (c.shape[0], 32)).astype(np.float32)).to(dtype)
    run_pool(c, 1, (12, 12, 12), 3, 2, 1, 1, x, dtype, ref, 195, "ties")


def test_maxpool_rows_without_inputs_and_empty_sides():
    # a synthetic map: rows with no entry give 0 and winner 255
    r = W.rng(196)
    n_in, M, K, C = 300, 1000, 8, 32
    nbr = np.where(r.random((K, M)) < 0.2, r.integers(0, n_in, (K, M)), -1).astype(np.int32)
    nbr[:, :50] = -1
    x = torch.from_numpy(r.standard_normal((n_in, C)).astype(np.float32))
    out, argk = spc.sparse_maxpool_fwd(cuda(x), cuda(np.ascontiguousarray(nbr.T)), M)
    ro, ra = P.maxpool_fwd(x, nbr)
    assert np.array_equal(exact(out), ro) and np.array_equal(host(argk), ra)
    assert (host(argk)[:50] == P.NO_ARG).all() and (exact(out)[:50] == 0).all()
    # no input rows at all: every output is 0 with no winner
    empty = torch.empty((0, C), dtype=torch.float32, device="cuda")
    out, argk = spc.sparse_maxpool_fwd(empty, cuda(np.full((M, K), -1, np.int32)), M)
    assert (exact(out) == 0).all() and (host(argk) == P.NO_ARG).all()
    # no output rows: the backward leaves every input gradient 0
    din = spc.sparse_maxpool_bwd(torch.empty((0, C), device="cuda"), torch.empty((0, C), dtype=torch.uint8,
                                 device="cuda"), cuda(np.full((n_in, K), -1, np.int32)), n_in)
    assert (exact(din) == 0).all()


def test_maxpool_errors():
    x = torch.zeros((10, 24), device="cuda")
    with pytest.raises(spc.SpcError) as e:
        spc.sparse_maxpool_fwd(x, torch.zeros((4, 8), dtype=torch.int32, device="cuda"), 4)
    assert e.value.status == spc.binding.SPC_ERR_UNSUPPORTED
    x = torch.zeros((10, 32), device="cuda")
    with pytest.raises(spc.SpcError) as e:
        spc.sparse_maxpool_fwd(x, torch.zeros((4, 255), dtype=torch.int32, device="cuda"), 4)
    assert e.value.status == spc.binding.SPC_ERR_UNSUPPORTED
    # a row's 16-byte chunks must fit one wave: at most 256 fp32 channels
    x = torch.zeros((10, 272), device="cuda")
    with pytest.raises(spc.SpcError) as e:
        spc.sparse_maxpool_fwd(x, torch.zeros((4, 8), dtype=torch.int32, device="cuda"), 4)
    assert e.value.status == spc.binding.SPC_ERR_UNSUPPORTED


@pytest.mark.parametrize("k,s,p", [(3, 2, 1), (2, 2, 0)])
def test_workload_maxpool_lidar_fp16(k, s, p):
    w = W.workload("strided_k3s2_f16_lidar120k")
    ref = O.strided_kmap(w.coords, w.batch, w.shape, k, s, p, 1)
    run_pool(w.coords, w.batch, w.shape, k, s, p, 1, w.feats, w.dtype, ref, 197, w.name)
