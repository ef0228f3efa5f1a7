"""CPU oracle for the Sampling-VT view transform.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP implementation.  ``oracle.multilevel`` holds the multi-level
(feature-pyramid) variant, ``oracle.lift_splat`` the push view transform,
``oracle.deform_agg`` the multi-camera deformable aggregation and
``oracle.brute_force`` the scalar checkers.
"""
from .sampling_vt import (EDGE_EPS_PX, bilinear_sample, bilinear_taps, height_sum, in_view_mask,  # noqa: F401
                          near_edge_mask, oracle_backward, oracle_forward, project,
                          tensorized_intermediates, valid_camera_mean, voxel_grid)
