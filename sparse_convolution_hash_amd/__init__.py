"""MI355X-native sparse 3-D convolution on voxel coordinate sets.

The compute lives in ``libspc.so`` (hand-written HIP kernels for gfx950
behind the C ABI of ``include/spc.h``); this package only binds it.
"""

from .binding import (  # noqa: F401
    EXPORTS,
    SpcError,
    build_kmap,
    calibrate_mfma,
    conv_bwd_filter,
    conv_bwd_filter_noalloc,
    conv_bwd_input,
    conv_fwd_dev_rows,
    conv_fwd_fused,
    conv_fwd_wt,
    gather_by_voxel_id,
    lib,
    make_geom,
    out_shape,
    strided_out_bound,
    point_to_voxel,
    sparse_conv_fwd,
    sparse_inverse_conv_fwd,
    sparse_maxpool_bwd,
    sparse_maxpool_fwd,
    subm_conv_fwd,
    transpose_weight,
    version,
)
