"""MI355X-native exact dense Sampling-VT (camera -> BEV view transform).

The operator runs in libflashbev.so (HIP kernels for gfx950 behind a C ABI,
declared in include/flashbev.h).  ``camera_bev_view_amd.ops`` is the thin
PyTorch binding; ``camera_bev_view_amd.workloads`` draws seeded synthetic
inputs.  Importing the package does not load the library; the first call
does, and fails loudly if it has not been built.
"""
__all__ = ["ops", "workloads", "build"]
