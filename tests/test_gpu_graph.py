"""HIP graph capture of a SubM layer step (kernel map, forward, k=1 layer,
dinput, dfilter): the library launches only kernels on the caller's stream
(no memsets, allocations or host waits on this path), so the step captures
as one graph.  Every replay, with eager work and synchronisations between
replays, must equal the eager step bit for bit (the kernels are
deterministic)."""

import numpy as np
import pytest
import torch

import sparse_convolution_hash_amd as spc
import workloads as W
from tests.parity import cuda

pytestmark = pytest.mark.gpu


def step(c, batch, shape, x, w, w1, g):
    km = spc.build_kmap(c, batch, shape, 3, orders=True)
    y = spc.subm_conv_fwd(x, w, None, km["nbr"], km["order"])
    z = spc.subm_conv_fwd(y, w1, None, None)
    din = spc.conv_bwd_input(g, w, km["nbr"], True, c.shape[0], km["order"])
    dw, db = spc.conv_bwd_filter(x, g, 27, km["pair_ptr"], km["pair_in"], km["pair_out"], want_dbias=True)
    return [km["nbr"], km["order"], km["pair_ptr"], y, z, din, dw, db]


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_subm_step_graph_replays_equal_eager(dtype):
    cc = W.tiny_grid(W.rng(240), 24, 0.2, 2)
    t = W.small_layer(240, cc, 32, 32, 27, dtype)
    c, x, w, g = cuda(cc), cuda(t["feats"]), cuda(t["weight"]), cuda(t["grad"])
    w1 = cuda(W.small_layer(241, cc, 32, 32, 1, dtype)["weight"])
    print(f"graph capture n={cc.shape[0]} {dtype}", flush=True)
    eager = step(c, 2, (24, 24, 24), x, w, w1, g)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm the allocator on the capture stream
        step(c, 2, (24, 24, 24), x, w, w1, g)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step(c, 2, (24, 24, 24), x, w, w1, g)
    for rep in range(3):
        for o in outs:
            o.fill_(-7)  # the replay must rewrite every output
        graph.replay()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(outs, eager)):
            assert torch.equal(a, b), f"replay {rep}: output {k} differs from the eager step"
        # eager work between replays
        spc.subm_conv_fwd(x, w, None, eager[0], eager[1])
        torch.cuda.synchronize()


def full_step(c, batch, shape, x, w, w1, g, ws, gs, cap):
    """Both layers of a step: the SubM layer as above, and the strided layer
    over a map that leaves its count on the device (no host wait anywhere)."""
    outs = step(c, batch, shape, x, w, w1, g)
    ks = spc.build_kmap(c, batch, shape, 3, 2, 1, 1, subm=False, orders=True, out_cap=cap, device_count=True)
    ys = spc.conv_fwd_dev_rows(x, ws, None, ks["nbr"], ks["n_out_dev"], cap, ks["order"])
    dins = spc.conv_bwd_input(gs, ws, ks["nbr_in"], False, c.shape[0], ks["order_in"])
    dws, _ = spc.conv_bwd_filter(x, gs, 27, ks["pair_ptr"], ks["pair_in"], ks["pair_out"])
    return outs + [ks["n_out_dev"], ks["out_coords"], ks["nbr"], ks["order"], ks["nbr_in"], ks["pair_ptr"], ys,
                   dins, dws]


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_full_step_graph_replays_equal_eager(dtype):
    # the whole step, strided layer included, captures as one graph once the
    # strided map leaves its count on the device; every replay equals the
    # eager step (rows past the count M are not compared: nothing writes them)
    cc = W.tiny_grid(W.rng(242), 24, 0.2, 2)
    shape = (24, 24, 24)
    t = W.small_layer(242, cc, 32, 32, 27, dtype)
    c, x, w, g = cuda(cc), cuda(t["feats"]), cuda(t["weight"]), cuda(t["grad"])
    w1 = cuda(W.small_layer(243, cc, 32, 32, 1, dtype)["weight"])
    cap = spc.strided_out_bound(cc.shape[0], 2, shape, 3, 2, 1, 1)
    ws = cuda(W.small_layer(244, cc, 32, 64, 27, dtype)["weight"])
    gs = cuda(W.grad_for(W.rng(245), cap, 64, dtype))
    args = (c, 2, shape, x, w, w1, g, ws, gs, cap)
    print(f"full-step graph capture n={cc.shape[0]} cap={cap} {dtype}", flush=True)
    eager = full_step(*args)
    torch.cuda.synchronize()
    M = int(eager[8].item())
    # the eager async step agrees with the waiting map and host-row forward
    ref = spc.build_kmap(c, 2, shape, 3, 2, 1, 1, subm=False, orders=True)
    assert ref["n_out"] == M
    assert torch.equal(eager[10][:M], ref["nbr"])
    assert torch.equal(eager[14][:M], spc.sparse_conv_fwd(x, ws, None, ref["nbr"], M, ref["order"]))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm the allocator on the capture stream
        full_step(*args)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = full_step(*args)
    rows = {9: M, 10: M, 11: M, 14: M}  # outputs with capacity rows: compare the first M
    for rep in range(3):
        for o in outs:
            o.fill_(-7)  # the replay must rewrite every output
        graph.replay()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(outs, eager)):
            n = rows.get(k)
            assert torch.equal(a[:n] if n is not None else a, b[:n] if n is not None else b), \
                f"replay {rep}: output {k} differs from the eager step"
        # eager work between replays
        spc.subm_conv_fwd(x, w, None, eager[0], eager[1])
        torch.cuda.synchronize()
