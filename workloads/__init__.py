"""Seeded synthetic inputs for the sparse-convolution workloads.

This package only draws random inputs (coordinates, features, weights,
gradients). It holds none of the convolution or kernel-map arithmetic, so both
the CPU oracle's tests and the HIP path's tests and benchmark can use it
without sharing any of the method.
"""

from .generators import (  # noqa: F401
    WORKLOAD_NAMES,
    Workload,
    LIDAR_VOXEL,
    grad_for,
    lidar_points,
    lidar_scene,
    mesh_shells,
    random_block,
    rng,
    small_layer,
    tiny_grid,
    uniform_grid,
    workload,
)
