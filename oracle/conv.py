"""Oracle convolution arithmetic (test infrastructure only; see the package docstring).

All sums run in float64 on the exact values of the (already quantised)
fp32 / fp16 / bf16 inputs.  ``nbr`` is always the output-stationary map
``[K, n_out]`` (the submanifold ``nbr`` or the strided ``nbr_out``), and the
weight layout is ``[K, Cin, Cout]`` (MLX ``sparse/conv.py`` page, ``SubMConv3d``).

Forward (MLX page, module docstring): ``out[o] = bias + sum_k feats[nbr[k][o]] @ W[k]``
over the offsets whose neighbour is present; an absent neighbour adds nothing.
dinput and dfilter are the adjoint and the weight derivative of that same sum
(the Hygon spconv-das README, "Public Interface Support": forward, dinput and
dfilter), written from it here rather than from any transposed map.
"""

from __future__ import annotations

import numpy as np
import torch


def f64(t) -> np.ndarray:
    """Exact float64 copy of a torch tensor or array of any float dtype."""
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def conv_fwd(feats, weight, bias, nbr) -> np.ndarray:
    """``out[o] = bias + sum_k feats[nbr[k][o]] @ W[k]`` (MLX page formula), fp64."""
    x, w = f64(feats), f64(weight)
    nbr = np.asarray(nbr)
    K, n_out = nbr.shape
    out = np.zeros((n_out, w.shape[2]), dtype=np.float64)
    if bias is not None:
        out += f64(bias)[None, :]
    for k in range(K):
        o = np.nonzero(nbr[k] >= 0)[0]
        out[o] += x[nbr[k][o]] @ w[k]
    return out


def conv_fwd_rows(feats, weight, bias, nbr, rows) -> np.ndarray:
    """The forward sum for selected output rows only, one row at a time."""
    x, w = f64(feats), f64(weight)
    b = None if bias is None else f64(bias)
    res = np.zeros((len(rows), w.shape[2]), dtype=np.float64)
    for r, o in enumerate(rows):
        acc = np.zeros(w.shape[2]) if b is None else b.copy()
        for k in range(nbr.shape[0]):
            i = nbr[k][o]
            if i >= 0:
                acc += x[i] @ w[k]
        res[r] = acc
    return res


def conv_bwd_input(dout, weight, nbr, n_in: int) -> np.ndarray:
    """Adjoint of ``conv_fwd`` in the features: ``din[i] = sum over (k, o) with
    nbr[k][o] = i of dout[o] @ W[k]^T``, fp64."""
    g, w = f64(dout), f64(weight)
    nbr = np.asarray(nbr)
    din = np.zeros((n_in, w.shape[1]), dtype=np.float64)
    for k in range(nbr.shape[0]):
        o = np.nonzero(nbr[k] >= 0)[0]
        i = nbr[k][o]
        # one offset maps distinct outputs to distinct inputs, so a plain
        # indexed add is exact here; np.add.at would give the same result
        assert np.unique(i).size == i.size
        din[i] += g[o] @ w[k].T
    return din


def conv_bwd_filter(feats, dout, nbr) -> np.ndarray:
    """Weight derivative of ``conv_fwd``: ``dW[k] = sum_o feats[nbr[k][o]]^T dout[o]``
    over present neighbours, fp64 ``[K, Cin, Cout]``."""
    x, g = f64(feats), f64(dout)
    nbr = np.asarray(nbr)
    dw = np.zeros((nbr.shape[0], x.shape[1], g.shape[1]), dtype=np.float64)
    for k in range(nbr.shape[0]):
        o = np.nonzero(nbr[k] >= 0)[0]
        dw[k] = x[nbr[k][o]].T @ g[o]
    return dw


def conv_bwd_bias(dout) -> np.ndarray:
    """Bias derivative: the column sum of ``dout``, fp64."""
    return f64(dout).sum(axis=0)


def conv_fwd_fused(feats, weight, bias, nbr, residual=None, relu=False) -> np.ndarray:
    """The fused conv-add-relu layer of the implicit-GEMM call on spconv
    TENSORRT_INT8_GUIDE.md ("Call Spconv Implicit GEMM with Calculated Scales
    and Bias"): ``act(bias + residual + sum_k feats[nbr[k][o]] @ W[k])`` with
    act = ReLU (``max(v, 0)``) or the identity, fp64."""
    x, w = f64(feats), f64(weight)
    nbr = np.asarray(nbr)
    out = np.zeros((nbr.shape[1], w.shape[2]), dtype=np.float64)
    if bias is not None:
        out += f64(bias)[None, :]
    if residual is not None:
        out += f64(residual)
    for k in range(nbr.shape[0]):
        o = np.nonzero(nbr[k] >= 0)[0]
        out[o] += x[nbr[k][o]] @ w[k]
    return np.maximum(out, 0.0) if relu else out


# ------------------------------------------------ inverse (upsampling) conv

# SparseInverseConv3d (spconv USAGE.md, the layer table and "Using
# SparseInverseConv for Inverse Sparse Operations"): an upsampling layer that
# reuses the kernel map saved by an earlier strided SparseConv3d (same
# indice_key) and writes its output on that layer's INPUT sites, so the result
# has the sites the downsampling started from.  Every pair (i, o) of offset k of
# the saved map (input row i = nbr[k][o] feeding output row o) carries the
# coarse row o back to the fine row i through the inverse layer's own W[k].
# ``nbr`` below is the saved strided map [K, M] as the forward conv used it.

def inverse_conv_fwd(feats, weight, bias, nbr, n_fine: int) -> np.ndarray:
    """``out[i] = bias + sum over (k, o) with nbr[k][o] = i of feats[o] @ W[k]``,
    fp64 ``[n_fine, Cout]``; ``feats`` is ``[M, Cin]`` on the coarse sites."""
    x, w = f64(feats), f64(weight)
    nbr = np.asarray(nbr)
    out = np.zeros((n_fine, w.shape[2]), dtype=np.float64)
    if bias is not None:
        out += f64(bias)[None, :]
    for k in range(nbr.shape[0]):
        o = np.nonzero(nbr[k] >= 0)[0]
        i = nbr[k][o]
        assert np.unique(i).size == i.size  # one offset pairs each fine row at most once
        out[i] += x[o] @ w[k]
    return out


def inverse_conv_bwd_input(dout, weight, nbr, n_coarse: int) -> np.ndarray:
    """Adjoint of ``inverse_conv_fwd`` in the coarse features:
    ``din[o] = sum_k dout[nbr[k][o]] @ W[k]^T`` over present pairs, fp64."""
    g, w = f64(dout), f64(weight)
    nbr = np.asarray(nbr)
    din = np.zeros((n_coarse, w.shape[1]), dtype=np.float64)
    for k in range(nbr.shape[0]):
        o = np.nonzero(nbr[k] >= 0)[0]
        din[o] += g[nbr[k][o]] @ w[k].T
    return din


def inverse_conv_bwd_filter(feats, dout, nbr) -> np.ndarray:
    """Weight derivative of ``inverse_conv_fwd``:
    ``dW[k] = sum_o feats[o]^T dout[nbr[k][o]]`` over present pairs, fp64."""
    x, g = f64(feats), f64(dout)
    nbr = np.asarray(nbr)
    dw = np.zeros((nbr.shape[0], x.shape[1], g.shape[1]), dtype=np.float64)
    for k in range(nbr.shape[0]):
        o = np.nonzero(nbr[k] >= 0)[0]
        dw[k] = x[o].T @ g[nbr[k][o]]
    return dw


def max_rel_err(got, ref) -> float:
    """Parity measure of every floating-point comparison: ``max|got - ref| /
    max|ref|`` over all elements, in float64 (the bound a result must meet is
    ``max|err| <= tol * max|ref|``).  The shapes must be equal (no
    broadcasting).  0 for empty arrays; for an all-zero ``ref`` the plain
    ``max|got - ref|``; ``inf`` when ``got`` holds a NaN where ``ref`` does not
    (NaN at the same place in both counts as equal)."""
    g, r = f64(got), f64(ref)
    if g.shape != r.shape:
        raise ValueError(f"max_rel_err: shapes differ, got {g.shape} vs ref {r.shape}")
    if r.size == 0:
        return 0.0
    both_nan = np.isnan(g) & np.isnan(r)
    diff = np.abs(np.where(both_nan, 0.0, g - r))
    if np.isnan(diff).any():
        return float("inf")
    scale = np.abs(np.where(np.isnan(r), 0.0, r)).max()
    err = diff.max()
    return float(err / scale) if scale > 0 else float(err)
