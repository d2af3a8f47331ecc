"""Shared helpers of the GPU parity tests: move seeded inputs to the GPU, run
the library through its binding, and compare with the oracle."""

import numpy as np
import torch

from oracle import conv as OC

# tolerances on max|gpu - ref| / max|ref|
TOL = {torch.float32: 1e-4, torch.float16: 1e-2, torch.bfloat16: 1e-2}
TOL_DW = 1e-4      # dW and dbias are fp32 outputs


def dev():
    return torch.device("cuda:0")


def cuda(t):
    if isinstance(t, np.ndarray):
        t = torch.from_numpy(np.ascontiguousarray(t))
    return t.contiguous().to(dev())


def host(t):
    return t.detach().cpu().numpy()


def assert_close(got, ref, tol, what=""):
    err = OC.max_rel_err(got, ref)
    assert err <= tol, f"{what}: max|err|/max|ref| = {err:.3e} > {tol:.0e}"
    return err


def pairs_equal(res, ref_ptr, ref_in, ref_out):
    """CSR pair lists from the GPU (first ptr[K] entries) equal the oracle's."""
    ptr = host(res["pair_ptr"])
    assert np.array_equal(ptr, ref_ptr), "pair_ptr differs"
    P = int(ptr[-1])
    assert np.array_equal(host(res["pair_in"][:P]), ref_in), "pair_in differs"
    assert np.array_equal(host(res["pair_out"][:P]), ref_out), "pair_out differs"
