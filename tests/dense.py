"""Dense-tensor helpers for the oracle pins: scatter voxels into a dense NCDHW
grid and run torch's own conv3d on it (a library routine independent of the
oracle's per-offset sums)."""

import numpy as np
import torch
import torch.nn.functional as F


def densify(coords, values, batch, shape, fill=0.0):
    """[N, C] values at (b, z, y, x) rows -> float64 [B, C, Z, Y, X], ``fill`` elsewhere."""
    v = torch.as_tensor(np.asarray(values), dtype=torch.float64)
    C = v.shape[1]
    d = torch.full((batch, C) + tuple(shape), fill, dtype=torch.float64)
    c = torch.as_tensor(np.asarray(coords, dtype=np.int64))
    if c.shape[0]:
        d[c[:, 0], :, c[:, 1], c[:, 2], c[:, 3]] = v
    return d


def sample(dense, coords):
    """Read a dense [B, C, Z, Y, X] tensor at (b, z, y, x) rows -> [N, C]."""
    c = torch.as_tensor(np.asarray(coords, dtype=np.int64))
    return dense[c[:, 0], :, c[:, 1], c[:, 2], c[:, 3]]


def torch_weight(weight, ksize):
    """[K, Cin, Cout] -> conv3d layout [Cout, Cin, kz, ky, kx]."""
    w = torch.as_tensor(np.asarray(weight), dtype=torch.float64)
    K, cin, cout = w.shape
    return w.reshape(ksize, ksize, ksize, cin, cout).permute(4, 3, 0, 1, 2).contiguous()


def dense_conv(coords, feats, weight, bias, batch, shape, ksize, stride=1, pad=None, dil=1):
    x = densify(coords, feats, batch, shape)
    b = None if bias is None else torch.as_tensor(np.asarray(bias), dtype=torch.float64)
    if pad is None:
        pad = ksize // 2
    return F.conv3d(x, torch_weight(weight, ksize), b, stride=stride, padding=pad, dilation=dil)


def dense_conv_transpose(coarse_coords, coarse_feats, weight, bias, batch, coarse_shape, fine_shape, ksize,
                         stride, pad, dil=1):
    """torch's conv_transpose3d of the coarse voxels scattered into a dense grid,
    with the output padding that makes its extent exactly ``fine_shape``."""
    x = densify(coarse_coords, coarse_feats, batch, coarse_shape)
    w = torch.as_tensor(np.asarray(weight), dtype=torch.float64)
    K, cin, cout = w.shape
    w = w.reshape(ksize, ksize, ksize, cin, cout).permute(3, 4, 0, 1, 2).contiguous()  # [Cin, Cout, kz, ky, kx]
    b = None if bias is None else torch.as_tensor(np.asarray(bias), dtype=torch.float64)
    op = tuple(f - ((c - 1) * stride - 2 * pad + dil * (ksize - 1) + 1) for f, c in zip(fine_shape, coarse_shape))
    return F.conv_transpose3d(x, w, b, stride=stride, padding=pad, output_padding=op, dilation=dil)
