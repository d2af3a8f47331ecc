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


def hygon_check(got, ref, cin, cout, fp32: bool, what=""):
    """Secondary check, the acceptance test of the Hygon spconv-das README
    (its public test-suite table): fp32 outputs pass torch.allclose with
    atol = rtol = 1e-4; fp16 / bf16 runs pass when the L2 norm of the error is
    below 10 * max(1, max(Cin, Cout) / 16).  Our reference is the fp64 oracle.
    Returns the L2 norm of the error."""
    g = torch.as_tensor(OC.f64(got))
    r = torch.as_tensor(OC.f64(ref))
    l2 = float(torch.linalg.vector_norm(g - r))
    if fp32:
        assert torch.allclose(g, r, atol=1e-4, rtol=1e-4), f"{what}: fails allclose(atol=rtol=1e-4)"
    else:
        bound = 10 * max(1.0, max(cin, cout) / 16)
        assert l2 < bound, f"{what}: L2 error {l2:.3g} >= {bound:g}"
    print(f"{what}: L2 error {l2:.3g}", flush=True)
    return l2
