"""ctypes loader for libflashbev.so (the C ABI declared in include/flashbev.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation of the operator.
"""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libflashbev.so")

FBEV_OK = 0
FBEV_ERR_INVALID_ARGUMENT = 1
FBEV_ERR_UNSUPPORTED = 2
FBEV_ERR_DEVICE = 3
FBEV_DTYPE_F32 = 0
FBEV_DTYPE_BF16 = 1
FBEV_MAX_CAMERAS = 64
FBEV_MAX_LEVELS = 4
ABI_VERSION = 8
FBEV_MAX_KEYPOINTS = 256
FBEV_NOALLOC_SCRATCH_BYTES = 4 << 20

EXPORTED = ("fbev_forward", "fbev_backward", "fbev_forward_levels", "fbev_backward_levels", "fbev_lss_forward",
            "fbev_lss_backward", "fbev_deform_forward", "fbev_deform_backward_workspace", "fbev_deform_backward",
            "fbev_backward_cameras_workspace",
            "fbev_backward_cameras", "fbev_backward_cameras_noalloc", "fbev_forward_temporal", "fbev_backward_temporal", "fbev_status_string",
            "fbev_last_error", "fbev_abi_version")


class FeatDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("N", ctypes.c_int32), ("C", ctypes.c_int32),
                ("H", ctypes.c_int32), ("W", ctypes.c_int32)]


class BevRange(ctypes.Structure):
    _fields_ = [("x_min", ctypes.c_float), ("x_max", ctypes.c_float), ("y_min", ctypes.c_float),
                ("y_max", ctypes.c_float), ("z_min", ctypes.c_float), ("z_max", ctypes.c_float)]


class FlashBevError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libflashbev status {status}: {message}")
        self.status = status


_lock = threading.Lock()
_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Open libflashbev.so once and declare its signatures."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise FlashBevError(-1, f"{path} is not built; run `python -m camera_bev_view_amd.build`")
        lib = ctypes.CDLL(path)
        vp, f32p = ctypes.c_void_p, ctypes.c_void_p
        lib.fbev_forward.argtypes = [vp, ctypes.c_int, FeatDesc, f32p, f32p, f32p, BevRange,
                                     ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, f32p, vp, vp]
        lib.fbev_forward.restype = ctypes.c_int
        lib.fbev_backward.argtypes = [f32p, FeatDesc, f32p, f32p, f32p, BevRange,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, f32p, vp]
        lib.fbev_backward.restype = ctypes.c_int
        i32p = ctypes.POINTER(ctypes.c_int32)
        lib.fbev_forward_levels.argtypes = [vp, ctypes.c_int, FeatDesc, ctypes.c_int32, i32p, f32p, f32p, f32p,
                                            BevRange, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, f32p, vp, vp]
        lib.fbev_forward_levels.restype = ctypes.c_int
        lib.fbev_backward_levels.argtypes = [f32p, FeatDesc, ctypes.c_int32, i32p, f32p, f32p, f32p, BevRange,
                                             ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, f32p, vp]
        lib.fbev_backward_levels.restype = ctypes.c_int
        i32, f32 = ctypes.c_int32, ctypes.c_float
        lib.fbev_lss_forward.argtypes = [f32p, f32p, FeatDesc, i32, f32, f32, f32p, f32p, f32p, BevRange, i32, i32,
                                         f32p, vp]
        lib.fbev_lss_forward.restype = ctypes.c_int
        lib.fbev_lss_backward.argtypes = [f32p, f32p, f32p, FeatDesc, i32, f32, f32, f32p, f32p, f32p, BevRange, i32,
                                          i32, f32p, f32p, vp]
        lib.fbev_lss_backward.restype = ctypes.c_int
        lib.fbev_deform_forward.argtypes = [f32p, FeatDesc, f32p, f32p, f32p, f32p, f32p, f32p, i32, i32, f32p, vp]
        lib.fbev_deform_forward.restype = ctypes.c_int
        lib.fbev_deform_backward_workspace.argtypes = [FeatDesc, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
        lib.fbev_deform_backward_workspace.restype = ctypes.c_int
        lib.fbev_deform_backward.argtypes = [f32p, f32p, FeatDesc, f32p, f32p, f32p, f32p, f32p, f32p, i32, i32, f32p,
                                             f32p, f32p, f32p, vp, ctypes.c_size_t, vp]
        lib.fbev_deform_backward.restype = ctypes.c_int
        lib.fbev_backward_cameras_workspace.argtypes = [FeatDesc, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
        lib.fbev_backward_cameras_workspace.restype = ctypes.c_int
        lib.fbev_backward_cameras.argtypes = [f32p, f32p, FeatDesc, f32p, f32p, f32p, BevRange, i32, i32, i32, f32p,
                                              f32p, f32p, vp, ctypes.c_size_t, vp]
        lib.fbev_backward_cameras.restype = ctypes.c_int
        lib.fbev_backward_cameras_noalloc.argtypes = [f32p, f32p, FeatDesc, f32p, f32p, f32p, BevRange, i32, i32, i32,
                                                      f32p, f32p, f32p, vp]
        lib.fbev_backward_cameras_noalloc.restype = ctypes.c_int
        lib.fbev_forward_temporal.argtypes = [vp, ctypes.c_int, FeatDesc, f32p, f32p, f32p, BevRange, i32, i32, i32,
                                              f32p, i32, f32p, f32p, vp, vp]
        lib.fbev_forward_temporal.restype = ctypes.c_int
        lib.fbev_backward_temporal.argtypes = [f32p, FeatDesc, f32p, f32p, f32p, BevRange, i32, i32, i32, i32, f32p,
                                               f32p, f32p, vp]
        lib.fbev_backward_temporal.restype = ctypes.c_int
        lib.fbev_status_string.argtypes = [ctypes.c_int]
        lib.fbev_status_string.restype = ctypes.c_char_p
        lib.fbev_last_error.argtypes = []
        lib.fbev_last_error.restype = ctypes.c_char_p
        lib.fbev_abi_version.argtypes = []
        lib.fbev_abi_version.restype = ctypes.c_int32
        got = lib.fbev_abi_version()
        if got != ABI_VERSION:
            raise FlashBevError(-1, f"{path} reports ABI {got}, this binding expects {ABI_VERSION}; rebuild it")
        _lib = lib
        return lib


def check(status: int) -> None:
    """Raise FlashBevError for a non-OK status, with the library's message."""
    if status != FBEV_OK:
        lib = load()
        raise FlashBevError(status, f"{lib.fbev_status_string(status).decode()}: {lib.fbev_last_error().decode()}")


def feat_desc(B: int, N: int, C: int, H: int, W: int) -> FeatDesc:
    return FeatDesc(B, N, C, H, W)


def bev_range(rng6) -> BevRange:
    return BevRange(*(float(v) for v in rng6))


def int32_array(values):
    """A ctypes int32 array (host memory) of ``values``, or None when empty."""
    values = [int(v) for v in values]
    return (ctypes.c_int32 * len(values))(*values) if values else None
