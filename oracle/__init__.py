"""CPU oracle for sparse 3-D convolution on voxel coordinate sets.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow reference that the
HIP library is checked against.  Only the test suite, ``__graft_entry__.smoke``
and the ``cpu_baseline`` leg of ``bench.py`` may import it; the library itself
never calls it and has no CPU fallback.  It shares no code with the HIP path.

* ``kmap``  -- kernel maps: the submanifold ``[K^3, N]`` neighbour map by sorted
  keys and binary search, and the strided output coordinates, maps and pair
  lists written out from their definition.
* ``conv``  -- forward, dinput, dfilter and dbias as per-offset fp64 sums, and
  the inverse (upsampling) convolution on a saved strided map with its
  dinput and dfilter.
* ``pool``  -- sparse max pooling over a strided map, forward (max and winning
  offset) and backward.
* ``voxel`` -- point-cloud voxelisation (points to voxels, coordinates, counts
  and per-point voxel ids) by one sequential pass over the points.

Every function cites the passage it follows.  Pins that tie it to the pages
and to mathematics live in ``tests/test_oracle_*.py``.
"""

from . import conv, kmap, pool, voxel  # noqa: F401
