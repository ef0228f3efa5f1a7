"""CPU: the C-ABI library loads, exports what include/flashbev.h declares, and
rejects bad arguments on the host before anything reaches a device."""
import ctypes
import os
import re
import subprocess

import pytest

from camera_bev_view_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashbev.h")
RNG = (-50.0, 50.0, -50.0, 50.0, -5.0, 3.0)
FAKE = 0x10000          # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+(fbev_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_declarations_match_binding():
    assert declared_functions() == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True, check=True)
    syms = {line.split()[-1] for line in out.stdout.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in syms, name
        assert getattr(lib, name) is not None


def test_version_and_status_strings(lib):
    assert lib.fbev_abi_version() == _lib.ABI_VERSION
    assert lib.fbev_status_string(0) == b"ok"
    assert lib.fbev_status_string(1) == b"invalid argument"
    assert lib.fbev_status_string(2) == b"unsupported"
    assert lib.fbev_status_string(3) == b"device error"


def fwd(lib, feat=FAKE, dtype=0, desc=(1, 6, 64, 16, 44), K=FAKE, R=FAKE, t=FAKE, rng=RNG, X=8, Y=8, Z=4,
        out=FAKE, counts=None):
    return lib.fbev_forward(feat, dtype, _lib.feat_desc(*desc), K, R, t, _lib.bev_range(rng), X, Y, Z, out, counts,
                            None)


def bwd(lib, grad=FAKE, desc=(1, 6, 64, 16, 44), K=FAKE, R=FAKE, t=FAKE, rng=RNG, X=8, Y=8, Z=4, gF=FAKE):
    return lib.fbev_backward(grad, _lib.feat_desc(*desc), K, R, t, _lib.bev_range(rng), X, Y, Z, gF, None)


@pytest.mark.parametrize("kwargs,status,msg", [
    (dict(desc=(-1, 6, 64, 16, 44)), 1, "negative feature size"),
    (dict(desc=(1, 6, 64, -16, 44)), 1, "negative feature size"),
    (dict(X=-1), 1, "negative grid size"),
    (dict(Z=70000), 1, "grid size above"),
    (dict(desc=(1, 65, 64, 16, 44)), 1, "exceeds FBEV_MAX_CAMERAS"),
    (dict(rng=(10.0, -10.0, -50.0, 50.0, -5.0, 3.0)), 1, "finite min < max"),
    (dict(rng=(-50.0, 50.0, 0.0, 0.0, -5.0, 3.0)), 1, "finite min < max"),
    (dict(rng=(-50.0, float("inf"), -50.0, 50.0, -5.0, 3.0)), 1, "finite min < max"),
    (dict(rng=(-50.0, 50.0, -50.0, 50.0, float("nan"), 3.0)), 1, "finite min < max"),
    (dict(K=None), 1, "K, R and t"),
    (dict(t=None), 1, "K, R and t"),
    (dict(feat=None), 1, "features is NULL"),
    (dict(out=None), 1, "out is NULL"),
    (dict(dtype=7), 2, "unknown dtype"),
    (dict(dtype=1, desc=(1, 6, 63, 16, 44)), 2, "even C"),
    (dict(feat=FAKE + 2), 2, "4-byte aligned"),
    (dict(desc=(1, 64, 4096, 128, 128)), 2, "limit 2^31"),
])
def test_forward_validation(lib, kwargs, status, msg):
    assert fwd(lib, **kwargs) == status
    assert msg in lib.fbev_last_error().decode()


@pytest.mark.parametrize("kwargs,status,msg", [
    (dict(desc=(1, 6, -64, 16, 44)), 1, "negative feature size"),
    (dict(Y=-3), 1, "negative grid size"),
    (dict(desc=(1, 100, 64, 16, 44)), 1, "exceeds FBEV_MAX_CAMERAS"),
    (dict(rng=(-50.0, 50.0, -50.0, 50.0, 3.0, -5.0)), 1, "finite min < max"),
    (dict(R=None), 1, "K, R and t"),
    (dict(gF=None), 1, "grad_features is NULL"),
    (dict(grad=None), 1, "grad_out is NULL"),
    (dict(desc=(1, 64, 2048, 128, 128)), 2, "limit 2^31"),
])
def test_backward_validation(lib, kwargs, status, msg):
    assert bwd(lib, **kwargs) == status
    assert msg in lib.fbev_last_error().decode()


def fwd_levels(lib, L=3, ratios=(1, 2, 4), desc=(1, 6, 64, 32, 88), feat=FAKE, X=8, Y=8, Z=4, out=FAKE):
    return lib.fbev_forward_levels(feat, 0, _lib.feat_desc(*desc), L, _lib.int32_array(ratios), FAKE, FAKE, FAKE,
                                   _lib.bev_range(RNG), X, Y, Z, out, None, None)


def bwd_levels(lib, L=3, ratios=(1, 2, 4), desc=(1, 6, 64, 32, 88), gF=FAKE):
    return lib.fbev_backward_levels(FAKE, _lib.feat_desc(*desc), L, _lib.int32_array(ratios), FAKE, FAKE, FAKE,
                                    _lib.bev_range(RNG), 8, 8, 4, gF, None)


@pytest.mark.parametrize("kwargs,status,msg", [
    (dict(L=0, ratios=()), 1, "feature levels outside"),
    (dict(L=5, ratios=(1, 2, 4, 8, 16)), 1, "feature levels outside"),
    (dict(L=2, ratios=()), 1, "ratios is NULL"),
    (dict(ratios=(2, 4, 8)), 1, "ratios[0] must be 1"),
    (dict(ratios=(1, 3, 4)), 1, "does not divide"),
    (dict(ratios=(1, 0, 4)), 1, "does not divide"),
    (dict(desc=(1, 6, 64, 32, 90), ratios=(1, 2, 4)), 1, "does not divide"),
    (dict(desc=(1, 22, 64, 32, 88)), 2, "cameras x levels exceeds 64"),
    (dict(feat=None), 1, "features is NULL"),
])
def test_forward_levels_validation(lib, kwargs, status, msg):
    assert fwd_levels(lib, **kwargs) == status
    assert msg in lib.fbev_last_error().decode()


@pytest.mark.parametrize("kwargs,status,msg", [
    (dict(L=9, ratios=(1,) * 9), 1, "feature levels outside"),
    (dict(ratios=(1, 2, 5)), 1, "does not divide"),
    (dict(gF=None), 1, "grad_features is NULL"),
])
def test_backward_levels_validation(lib, kwargs, status, msg):
    assert bwd_levels(lib, **kwargs) == status
    assert msg in lib.fbev_last_error().decode()


def test_empty_problems_return_ok_without_device_work(lib):
    # nothing to write: no launch happens, so these succeed on a host without a GPU
    assert fwd(lib, desc=(0, 6, 64, 16, 44), feat=None, K=None, R=None, t=None, out=None) == 0
    assert fwd(lib, X=0, out=None) == 0
    assert fwd(lib, desc=(1, 6, 0, 16, 44), out=None, counts=None) == 0
    assert bwd(lib, desc=(0, 6, 64, 16, 44), grad=None, gF=None, K=None, R=None, t=None) == 0
    assert bwd(lib, desc=(1, 6, 0, 16, 44), grad=None, gF=None) == 0
    assert fwd_levels(lib, desc=(0, 6, 64, 32, 88), feat=None, out=None) == 0
    assert fwd_levels(lib, L=1, ratios=(), X=0, out=None) == 0


def test_binding_refuses_missing_library(tmp_path):
    with pytest.raises(_lib.FlashBevError):
        _lib._lib_saved = _lib._lib
        try:
            _lib._lib = None
            _lib.load(str(tmp_path / "missing.so"))
        finally:
            _lib._lib = _lib._lib_saved
