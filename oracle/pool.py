"""Oracle sparse max pooling (test infrastructure only; see the package docstring).

SparseMaxPool3d (spconv USAGE.md, the layer table: a downsampling layer whose
dense version is ``nn.MaxPool3d``, keyed like a strided SparseConv3d; the
layer comparison there pairs it with MinkowskiEngine's MinkowskiMaxPooling)
gives every output site of the strided kernel map built with the pool's
kernel size, stride and padding the channel-wise maximum over the input rows
that map pairs it with.  ``nbr`` is that output-stationary map ``[K, M]``.

Readings where the pages are silent:

* ties go to the first maximum in offset order, k = (kz * k + ky) * k + kx,
  which is also the scan order of a dense max-pool window;
* the winning offset index is kept per (row, channel) for the backward, as
  uint8 (pool kernels have at most 255 offsets);
* an output row with no paired input (a strided map never makes one) is 0
  and has no winner;
* NaN inputs are outside the contract (the comparisons skip them).
"""

from __future__ import annotations

import numpy as np

from .conv import f64

NO_ARG = 255  # winner index of a row/channel with no paired input


def maxpool_fwd(feats, nbr):
    """``(out, argk)``: ``out[o][c] = max over present k of feats[nbr[k][o]][c]``
    (fp64 ``[M, C]``) and ``argk[o][c]`` the first offset reaching it (uint8)."""
    x = f64(feats)
    nbr = np.asarray(nbr)
    K, M = nbr.shape
    assert K <= NO_ARG
    out = np.full((M, x.shape[1]), -np.inf)
    argk = np.full((M, x.shape[1]), NO_ARG, dtype=np.uint8)
    for k in range(K):
        o = np.nonzero(nbr[k] >= 0)[0]
        v = x[nbr[k][o]]
        better = v > out[o]  # strictly greater: an equal later value never wins
        out[o] = np.where(better, v, out[o])
        argk[o] = np.where(better, np.uint8(k), argk[o])
    out[argk == NO_ARG] = 0.0
    return out, argk


def maxpool_bwd(dout, argk, nbr, n_in: int) -> np.ndarray:
    """``din`` fp64 ``[n_in, C]``: each output's gradient goes, channel by
    channel, to the input row that won that channel's maximum."""
    g = f64(dout)
    nbr = np.asarray(nbr)
    argk = np.asarray(argk)
    din = np.zeros((n_in, g.shape[1]), dtype=np.float64)
    o, c = np.nonzero(argk != NO_ARG)
    i = nbr[argk[o, c].astype(np.int64), o]
    np.add.at(din, (i, c), g[o, c])
    return din
