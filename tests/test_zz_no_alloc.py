"""The allocation-free dfilter (spc_conv_bwd_filter_noalloc) against the
workspace form (spc_conv_bwd_filter) it varies: two calls in a row on the
same GPU, the second with a smaller input, each compared with the workspace
form's result (bit for bit: the same kernels and segment count) and with the
oracle within the fp32 tolerance; plus its size limit.  Through the C ABI
(the ctypes binding)."""

import numpy as np
import pytest
import torch

import sparse_convolution_hash_amd as spc
import workloads as W
from oracle import conv as OC
from oracle import kmap as O
from tests.parity import TOL_DW, assert_close, cuda

pytestmark = pytest.mark.gpu


def _case(seed, side, fill, batch, cin, cout, dtype):
    c = W.tiny_grid(W.rng(seed), side, fill, batch)
    t = W.small_layer(seed, c, cin, cout, 27, dtype)
    km = spc.build_kmap(cuda(c), batch, (side,) * 3, 3)
    return c, t, km


def _both(t, km, K=27):
    x, g = cuda(t["feats"]), cuda(t["grad"])
    dw_ref, db_ref = spc.conv_bwd_filter(x, g, K, km["pair_ptr"], km["pair_in"], km["pair_out"], want_dbias=True)
    dw = torch.full_like(dw_ref, float("nan"))
    db = torch.full_like(db_ref, float("nan"))
    spc.conv_bwd_filter_noalloc(x, g, K, km["pair_ptr"], km["pair_in"], km["pair_out"], dw, db)
    torch.cuda.synchronize()
    return dw, db, dw_ref, db_ref


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
def test_noalloc_matches_workspace_form_twice(dtype):
    # a larger call, then a smaller one: the second must not see the first's scratch
    for seed, side, fill, batch, cin, cout in ((501, 24, 0.3, 2, 128, 128), (502, 9, 0.2, 1, 32, 48)):
        print(f"noalloc dfilter seed={seed} side={side} cin={cin} cout={cout} {dtype}", flush=True)
        c, t, km = _case(seed, side, fill, batch, cin, cout, dtype)
        dw, db, dw_ref, db_ref = _both(t, km)
        assert torch.equal(dw, dw_ref) and torch.equal(db, db_ref)
        nbr = O.subm_kmap(c, (side,) * 3, 3)
        assert_close(dw.cpu(), OC.conv_bwd_filter(t["feats"], t["grad"], nbr), TOL_DW, "dw")
        assert_close(db.cpu(), OC.conv_bwd_bias(t["grad"]), TOL_DW, "dbias")


def test_noalloc_identity_and_limit():
    # K = 1 with no pair lists (row i with row i), and a size beyond the scratch
    c = W.tiny_grid(W.rng(503), 10, 0.3, 1)
    t = W.small_layer(503, c, 64, 64, 1, torch.bfloat16)
    x, g = cuda(t["feats"]), cuda(t["grad"])
    ref, _ = spc.conv_bwd_filter(x, g, 1, None, None, None)
    dw = torch.empty_like(ref)
    spc.conv_bwd_filter_noalloc(x, g, 1, None, None, None, dw)
    torch.cuda.synchronize()
    assert torch.equal(dw, ref)
    big = torch.zeros((8, 256), dtype=torch.bfloat16, device="cuda")
    pp = torch.zeros(28, dtype=torch.int32, device="cuda")
    pi = torch.zeros(16, dtype=torch.int32, device="cuda")
    with pytest.raises(spc.SpcError) as e:
        spc.conv_bwd_filter_noalloc(big, big, 27, pp, pi, pi, torch.empty((27, 256, 256), device="cuda"))
    assert e.value.status == spc.binding.SPC_ERR_UNSUPPORTED and "scratch" in str(e.value)
