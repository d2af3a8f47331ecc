"""The C ABI without Python: tests/abi_c/abi_driver (a host program built
against include/spc.h and libspc.so only) builds a submanifold kernel map and
runs the fp32 forward; its map must equal the oracle's bit for bit and its
outputs must be within the fp32 tolerance."""

import os
import subprocess

import numpy as np
import pytest
import torch

import workloads as W
from oracle import conv as OC
from oracle import kmap as O

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "abi_c", "abi_driver")


def test_c_abi_driver_subm_layer(tmp_path):
    assert os.path.exists(EXE), "the C ABI driver is not built (run __graft_entry__.build())"
    shape, k, cin, cout = (20, 20, 20), 3, 32, 48
    c = W.tiny_grid(W.rng(280), shape[0], 0.25, 2)
    t = W.small_layer(280, c, cin, cout, k ** 3, torch.float32)
    n = c.shape[0]
    src, dst = tmp_path / "layer.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        np.array([n, cin, cout, 2, *shape, k], np.int32).tofile(f)
        c.astype(np.int32).tofile(f)
        for key in ("feats", "weight", "bias"):
            t[key].numpy().astype(np.float32).tofile(f)
    print(f"C ABI driver: n={n} {cin}->{cout} k={k}", flush=True)
    r = subprocess.run([EXE, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    raw = np.fromfile(dst, np.uint8)
    err = raw[:4].view(np.int32)[0]
    K = k ** 3
    nbr = raw[4:4 + n * K * 4].view(np.int32).reshape(n, K)
    out = raw[4 + n * K * 4:].view(np.float32).reshape(n, cout)
    ref = O.subm_kmap(c, shape, k)
    assert err == 0
    assert np.array_equal(nbr, ref.T)
    e = OC.max_rel_err(out, OC.conv_fwd(t["feats"], t["weight"], t["bias"], ref))
    assert e <= 1e-4, e
