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


def lss_fwd(lib, depth=FAKE, ctx=FAKE, desc=(1, 6, 64, 8, 22), D=41, d_min=4.0, d_step=1.0, K=FAKE, R=FAKE, t=FAKE,
            rng=RNG, X=8, Y=8, out=FAKE):
    return lib.fbev_lss_forward(depth, ctx, _lib.feat_desc(*desc), D, d_min, d_step, K, R, t, _lib.bev_range(rng), X, Y,
                                out, None)


def lss_bwd(lib, grad=FAKE, depth=FAKE, ctx=FAKE, desc=(1, 6, 64, 8, 22), D=41, d_min=4.0, d_step=1.0, rng=RNG,
            X=8, Y=8, gd=FAKE, gc=FAKE, K=FAKE):
    return lib.fbev_lss_backward(grad, depth, ctx, _lib.feat_desc(*desc), D, d_min, d_step, K, FAKE, FAKE,
                                 _lib.bev_range(rng), X, Y, gd, gc, None)


@pytest.mark.parametrize("kwargs,status,msg", [
    (dict(desc=(1, 6, -64, 8, 22)), 1, "negative size"),
    (dict(D=-1), 1, "negative size"),
    (dict(X=-2), 1, "negative grid size"),
    (dict(D=70000), 1, "size above"),
    (dict(desc=(1, 65, 64, 8, 22)), 1, "exceeds FBEV_MAX_CAMERAS"),
    (dict(rng=(10.0, -10.0, -50.0, 50.0, -5.0, 3.0)), 1, "x and y BEV ranges"),
    (dict(d_step=0.0), 1, "d_step > 0"),
    (dict(d_step=-1.0), 1, "d_step > 0"),
    (dict(d_min=float("nan")), 1, "finite d_min"),
    (dict(K=None), 1, "K, R and t"),
    (dict(out=None), 1, "out is NULL"),
    (dict(depth=None), 1, "depth is NULL"),
    (dict(ctx=None), 1, "context is NULL"),
    (dict(desc=(1, 64, 4096, 128, 128)), 2, "limit 2^31"),
])
def test_lss_forward_validation(lib, kwargs, status, msg):
    assert lss_fwd(lib, **kwargs) == status
    assert msg in lib.fbev_last_error().decode()


def test_lss_forward_ignores_the_z_range(lib):
    # the z fields of the range are unused (pillars): an empty z interval is not an error; the call
    # then fails only at the NULL check that follows
    assert lss_fwd(lib, rng=(-50.0, 50.0, -50.0, 50.0, 3.0, -5.0), out=None) == 1
    assert "out is NULL" in lib.fbev_last_error().decode()


@pytest.mark.parametrize("kwargs,status,msg", [
    (dict(D=-3), 1, "negative size"),
    (dict(d_step=float("inf")), 1, "d_step > 0"),
    (dict(gd=None), 1, "grad_depth is NULL"),
    (dict(gc=None), 1, "grad_context is NULL"),
    (dict(depth=None), 1, "depth and context"),
    (dict(grad=None), 1, "grad_out is NULL"),
    (dict(desc=(1, 64, 1024, 256, 256)), 2, "limit 2^31"),
])
def test_lss_backward_validation(lib, kwargs, status, msg):
    assert lss_bwd(lib, **kwargs) == status
    assert msg in lib.fbev_last_error().decode()


def test_lss_empty_problems_return_ok_without_device_work(lib):
    assert lss_fwd(lib, desc=(0, 6, 64, 8, 22), depth=None, ctx=None, K=None, R=None, t=None, out=None) == 0
    assert lss_fwd(lib, Y=0, out=None) == 0
    assert lss_fwd(lib, desc=(1, 6, 0, 8, 22), out=None) == 0
    assert lss_bwd(lib, desc=(0, 6, 64, 8, 22), grad=None, depth=None, ctx=None, gd=None, gc=None, K=None) == 0
    assert lss_bwd(lib, desc=(1, 6, 64, 0, 22), grad=None, depth=None, ctx=None, gd=None, gc=None) == 0


def dfwd(lib, feat=FAKE, desc=(1, 6, 64, 16, 44), K=FAKE, A=FAKE, D=FAKE, Wt=FAKE, Q=10, Kp=4, out=FAKE):
    return lib.fbev_deform_forward(feat, _lib.feat_desc(*desc), K, FAKE, FAKE, A, D, Wt, Q, Kp, out, None)


def dbwd(lib, grad=FAKE, feat=FAKE, desc=(1, 6, 64, 16, 44), A=FAKE, D=FAKE, Wt=FAKE, Q=10, Kp=4, gF=FAKE, gW=FAKE,
         gO=FAKE, gA=None, ws=FAKE, ws_bytes=1 << 30):
    return lib.fbev_deform_backward(grad, feat, _lib.feat_desc(*desc), FAKE, FAKE, FAKE, A, D, Wt, Q, Kp, gF, gW, gO,
                                    gA, ws, ws_bytes, None)


def deform_workspace(lib, desc=(1, 6, 64, 16, 44), Q=10, Kp=4):
    n = ctypes.c_size_t(12345)
    st = lib.fbev_deform_backward_workspace(_lib.feat_desc(*desc), Q, Kp, ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("kwargs,status,msg", [
    (dict(desc=(1, 6, -1, 16, 44)), 1, "negative size"),
    (dict(Q=-1), 1, "negative size"),
    (dict(Kp=-2), 1, "negative size"),
    (dict(Kp=257), 1, "FBEV_MAX_KEYPOINTS"),
    (dict(desc=(1, 65, 64, 16, 44)), 1, "exceeds FBEV_MAX_CAMERAS"),
    (dict(K=None), 1, "K, R and t"),
    (dict(out=None), 1, "out is NULL"),
    (dict(A=None), 1, "anchors is NULL"),
    (dict(D=None), 1, "offsets and weights"),
    (dict(Wt=None), 1, "offsets and weights"),
    (dict(feat=None), 1, "features is NULL"),
    (dict(desc=(1, 64, 4096, 128, 128)), 2, "limit 2^31"),
])
def test_deform_forward_validation(lib, kwargs, status, msg):
    assert dfwd(lib, **kwargs) == status
    assert msg in lib.fbev_last_error().decode()


@pytest.mark.parametrize("kwargs,status,msg", [
    (dict(Q=-3), 1, "negative size"),
    (dict(gF=None), 1, "grad_features is NULL"),
    (dict(gW=None), 1, "grad_weights is NULL"),
    (dict(gO=None), 1, "grad_offsets is NULL"),
    (dict(A=None), 1, "anchors is NULL"),
    (dict(D=None), 1, "offsets is NULL"),
    (dict(Wt=None), 1, "weights is NULL"),
    (dict(grad=None), 1, "features and grad_out"),
    (dict(feat=None), 1, "features and grad_out"),
    (dict(ws=None), 1, "workspace of 0 bytes given"),
    (dict(ws_bytes=100), 1, "workspace of 100 bytes given"),
    (dict(ws=FAKE + 8), 1, "16-byte aligned"),
    (dict(desc=(8, 64, 1, 2048, 2048)), 2, "feature pixels"),
    (dict(Q=1 << 24, Kp=64), 2, "gradient entries"),
])
def test_deform_backward_validation(lib, kwargs, status, msg):
    assert dbwd(lib, **kwargs) == status
    assert msg in lib.fbev_last_error().decode()


def test_deform_empty_problems_return_ok_without_device_work(lib):
    assert dfwd(lib, desc=(0, 6, 64, 16, 44), feat=None, K=None, A=None, D=None, Wt=None, out=None) == 0
    assert dfwd(lib, Q=0, A=None, D=None, Wt=None, out=None) == 0
    assert dfwd(lib, desc=(1, 6, 0, 16, 44), out=None) == 0
    assert dbwd(lib, desc=(0, 6, 64, 16, 44), grad=None, feat=None, A=None, D=None, Wt=None, gF=None, gW=None,
                gO=None, ws=None) == 0


def test_deform_workspace_size(lib):
    st, n = deform_workspace(lib)
    # counts and offsets per pixel, one count per query, 4 N Kp entries of 12 + 8 bytes per query, 256-byte parts
    npix, nq, ne = 6 * 16 * 44, 10, 10 * 4 * 6 * 4
    up = lambda x: -(-x // 256) * 256
    assert st == 0 and n == 2 * up(4 * npix) + up(4) + up(4 * nq) + up(12 * ne) + up(8 * ne)
    # nothing to gather: no workspace
    assert deform_workspace(lib, Q=0) == (0, 0)
    assert deform_workspace(lib, Kp=0) == (0, 0)
    assert deform_workspace(lib, desc=(1, 6, 0, 16, 44)) == (0, 0)
    assert deform_workspace(lib, desc=(0, 6, 64, 16, 44)) == (0, 0)
    assert deform_workspace(lib, Q=-1)[0] == 1
    assert deform_workspace(lib, Q=1 << 24, Kp=64)[0] == 2
    assert lib.fbev_deform_backward_workspace(_lib.feat_desc(1, 6, 64, 16, 44), 10, 4, None) == 1


def cbwd(lib, grad=FAKE, feat=FAKE, desc=(1, 6, 64, 16, 44), K=FAKE, rng=RNG, X=200, Y=200, Z=8, gK=FAKE, gR=FAKE,
         gt=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return lib.fbev_backward_cameras(grad, feat, _lib.feat_desc(*desc), K, FAKE, FAKE, _lib.bev_range(rng), X, Y, Z,
                                     gK, gR, gt, ws, ws_bytes, None)


def cam_workspace(lib, desc=(1, 6, 64, 16, 44), X=200, Y=200, Z=8):
    n = ctypes.c_size_t(12345)
    st = lib.fbev_backward_cameras_workspace(_lib.feat_desc(*desc), X, Y, Z, ctypes.byref(n))
    return st, n.value


def test_camera_workspace_size(lib):
    st, n = cam_workspace(lib)
    # fp64 dL/dP slices, 12 per camera and workgroup
    assert st == 0 and n > 0 and n % (8 * 6 * 12) == 0
    st0, n0 = cam_workspace(lib, Z=0)
    assert st0 == 0 and 0 < n0 < n
    assert cam_workspace(lib, desc=(1, 6, 0, 16, 44)) == (0, n0)
    assert cam_workspace(lib, desc=(0, 6, 64, 16, 44)) == (0, 0)
    assert cam_workspace(lib, desc=(1, 0, 64, 16, 44)) == (0, 0)
    assert cam_workspace(lib, X=-1)[0] == 1
    assert lib.fbev_backward_cameras_workspace(_lib.feat_desc(1, 6, 64, 16, 44), 200, 200, 8, None) == 1


@pytest.mark.parametrize("kwargs,status,msg", [
    (dict(desc=(1, 6, -1, 16, 44)), 1, "negative feature size"),
    (dict(Z=-1), 1, "negative grid size"),
    (dict(desc=(1, 65, 64, 16, 44)), 1, "exceeds FBEV_MAX_CAMERAS"),
    (dict(rng=(1.0, 1.0, -50.0, 50.0, -5.0, 3.0)), 1, "finite min < max"),
    (dict(K=None), 1, "K, R and t"),
    (dict(gK=None), 1, "grad_K, grad_R and grad_t"),
    (dict(gt=None), 1, "grad_K, grad_R and grad_t"),
    (dict(feat=None), 1, "features is NULL"),
    (dict(grad=None), 1, "grad_out is NULL"),
    (dict(feat=FAKE + 2), 2, "4-byte aligned"),
    (dict(ws=None), 1, "workspace"),
    (dict(ws_bytes=100), 1, "workspace"),
    (dict(ws=FAKE + 4), 1, "8-byte aligned"),
    (dict(desc=(1, 64, 4096, 128, 128)), 2, "limit 2^31"),
])
def test_camera_backward_validation(lib, kwargs, status, msg):
    assert cbwd(lib, **kwargs) == status
    assert msg in lib.fbev_last_error().decode()


def test_camera_empty_problems_return_ok_without_device_work(lib):
    assert cbwd(lib, desc=(0, 6, 64, 16, 44), grad=None, feat=None, K=None, gK=None, gR=None, gt=None, ws=None) == 0
    assert cbwd(lib, desc=(1, 0, 64, 16, 44), K=None, gK=None, gR=None, gt=None, ws=None) == 0


def tfwd(lib, feat=FAKE, desc=(1, 6, 64, 16, 44), X=200, Y=200, Z=8, prev=FAKE, Cp=64, ego=FAKE, out=FAKE):
    return lib.fbev_forward_temporal(feat, _lib.FBEV_DTYPE_F32, _lib.feat_desc(*desc), FAKE, FAKE, FAKE,
                                     _lib.bev_range(RNG), X, Y, Z, prev, Cp, ego, out, None, None)


def tbwd(lib, grad=FAKE, desc=(1, 6, 64, 16, 44), X=200, Y=200, Z=8, Cp=64, ego=FAKE, gF=FAKE, gP=FAKE, rng=RNG):
    return lib.fbev_backward_temporal(grad, _lib.feat_desc(*desc), FAKE, FAKE, FAKE, _lib.bev_range(rng), X, Y, Z, Cp,
                                      ego, gF, gP, None)


@pytest.mark.parametrize("kwargs,status,msg", [
    (dict(Cp=-1), 1, "negative Cp"),
    (dict(prev=None), 1, "prev_bev is NULL"),
    (dict(ego=None), 1, "ego is NULL"),
    (dict(out=None), 1, "out is NULL"),
    (dict(X=65536, Y=65536, Z=1), 2, "X*Y"),
    (dict(desc=(1, 6, 64, -16, 44)), 1, "negative feature size"),
])
def test_temporal_forward_validation(lib, kwargs, status, msg):
    assert tfwd(lib, **kwargs) == status
    assert msg in lib.fbev_last_error().decode()


@pytest.mark.parametrize("kwargs,status,msg", [
    (dict(Cp=-2), 1, "negative Cp"),
    (dict(gP=None), 1, "grad_prev is NULL"),
    (dict(ego=None), 1, "ego is NULL"),
    (dict(grad=None), 1, "grad_out is NULL"),
    (dict(gF=None), 1, "grad_features is NULL"),
    # 0.5 m x 10 m cells: a turn's inverse spans 1 + 20 cells along x, past the gather window
    (dict(X=200, Y=10), 2, "cell aspect ratio"),
    (dict(X=7, Y=200, rng=(-50.0, 50.0, -1.0, 1.0, -5.0, 3.0)), 2, "cell aspect ratio"),
])
def test_temporal_backward_validation(lib, kwargs, status, msg):
    assert tbwd(lib, **kwargs) == status
    assert msg in lib.fbev_last_error().decode()


def test_temporal_empty_problems_return_ok_without_device_work(lib):
    assert tfwd(lib, desc=(0, 6, 64, 16, 44), feat=None, prev=None, ego=None, out=None) == 0
    assert tfwd(lib, X=0, prev=None, ego=None, out=None) == 0
    assert tbwd(lib, desc=(0, 6, 64, 16, 44), grad=None, ego=None, gF=None, gP=None) == 0


NO_GPU_HOST = not os.path.exists("/dev/kfd")


@pytest.mark.skipif(not NO_GPU_HOST, reason="forces HIP's launch failure by having no device; needs a GPU-less host")
def test_launch_failure_maps_to_device_error(lib):
    """Valid arguments on a host without a GPU: validation passes, the HIP launch itself fails, and the
    call returns FBEV_ERR_DEVICE with HIP's reason in fbev_last_error (nothing is dereferenced)."""
    assert fwd(lib) == _lib.FBEV_ERR_DEVICE
    msg = lib.fbev_last_error().decode()
    assert msg.startswith("fbev_forward launch: ") and len(msg) > len("fbev_forward launch: ")
    assert bwd(lib) == _lib.FBEV_ERR_DEVICE
    assert lib.fbev_last_error().decode().startswith("fbev_backward launch: ")
    assert lib.fbev_status_string(_lib.FBEV_ERR_DEVICE) == b"device error"
    # a later valid-argument error replaces the text
    assert fwd(lib, X=-1) == _lib.FBEV_ERR_INVALID_ARGUMENT
    assert "negative grid size" in lib.fbev_last_error().decode()
