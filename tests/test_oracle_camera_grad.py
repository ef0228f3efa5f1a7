"""CPU: pins of the camera-gradient oracle (oracle.camera_grad).

What fixes it independently of oracle.camera_grad:
  * central finite differences of the forward oracle (oracle.sampling_vt) in
    every entry of K, R and t, on rigs with level and pitched cameras;
  * a hand-derived golden point: one yaw-0 camera, one cell, features that
    ramp along the image columns (channel 0) and rows (channel 1), so the
    output is u + 2 v and every partial derivative is written out from the
    camera-frame formulas u = f X_c / Z_c + c_x, v = f Y_c / Z_c + c_y;
  * two identical cameras that both see the cell: each gets half of the one-
    camera gradient (the valid-camera mean);
  * homogeneity: K -> s K and [R | t] -> s [R | t] leave every projection
    unchanged, so <K, dL/dK> = 0 and <R, dL/dR> + <t, dL/dt> = 0;
  * constant features give zero gradients.
Planted mistakes are each caught by these pins.
"""
import numpy as np
import pytest

import oracle.camera_grad as cg
import oracle.sampling_vt as svt
from camera_bev_view_amd import workloads as wl


def small_case(seed, N=6, C=3, H=7, W=11, X=12, Y=12, Z=3, pitch=0.0, rng6=(-12.0, 12.0, -12.0, 12.0, -1.5, 2.5)):
    K, R, t = wl.make_rig(70 + seed, 1, N, H, W, True, pitch_deg=pitch)
    g = np.random.default_rng(seed)
    F = g.standard_normal((1, N, C, H, W))
    G = g.standard_normal((1, C, X, Y))
    return F, K.astype(np.float64), R.astype(np.float64), t.astype(np.float64), rng6, X, Y, Z, G


def loss(F, K, R, t, rng6, X, Y, Z, G):
    r = svt.oracle_forward(F, K, R, t, rng6, X, Y, Z)
    return float((G * r["out"]).sum()), r["counts"]


def finite_differences(F, K, R, t, rng6, X, Y, Z, G, h=1e-6):
    """Central differences of <G, out> in every entry of K, R and t (counts must not change)."""
    _, c0 = loss(F, K, R, t, rng6, X, Y, Z, G)
    out = {}
    for name, arr in (("K", K), ("R", R), ("t", t)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(*arr.shape):
            step = h * max(1.0, abs(arr[idx]))
            ap, am = arr.copy(), arr.copy()
            ap[idx] += step
            am[idx] -= step
            args_p = {"K": K, "R": R, "t": t}
            args_m = {"K": K, "R": R, "t": t}
            args_p[name], args_m[name] = ap, am
            lp, cp = loss(F, args_p["K"], args_p["R"], args_p["t"], rng6, X, Y, Z, G)
            lm, cm = loss(F, args_m["K"], args_m["R"], args_m["t"], rng6, X, Y, Z, G)
            assert np.array_equal(cp, c0) and np.array_equal(cm, c0), f"mask changed under d{name}{idx}"
            num[idx] = (lp - lm) / (2 * step)
        out[name] = num
    return out


def _fd_pin(seed, pitch):
    F, K, R, t, rng6, X, Y, Z, G = small_case(seed, pitch=pitch)
    got = cg.oracle_camera_backward(G, F, K, R, t, rng6, X, Y, Z)
    num = finite_differences(F, K, R, t, rng6, X, Y, Z, G)
    for name in ("K", "R", "t"):
        ref = num[name]
        assert np.abs(ref).max() > 0
        err = np.abs(got[name] - ref).max()
        assert err <= 1e-5 * np.abs(ref).max(), f"d{name}: max |analytic - numeric| {err:.3e}"


def test_finite_differences_level_rig():
    _fd_pin(1, 0.0)


def test_finite_differences_pitched_rig():
    _fd_pin(2, -6.0)


def golden_setup(n_cams=1, C=2):
    H, W = 8, 22
    Kn, Rn, tn = (a.astype(np.float64) for a in wl.make_rig(0, 1, 1, H, W, False, jitter=False))
    K = np.repeat(Kn, n_cams, axis=1)
    R = np.repeat(Rn, n_cams, axis=1)
    t = np.repeat(tn, n_cams, axis=1)
    F = np.zeros((1, n_cams, C, H, W))
    F[:, :, 0] = np.arange(W)[None, :]          # column ramp: the sample is u
    F[:, :, 1] = np.arange(H)[:, None]          # row ramp: the sample is v
    rng6 = (5.5, 6.5, 0.0, 1.0, 0.5, 1.5)       # one cell, centre (6, 0.5, 1.0)
    G = np.array([1.0, 2.0]).reshape(1, 2, 1, 1)
    return F, K, R, t, rng6, G


def golden_expected():
    """Yaw-0 camera at (1, 0, 1.6) looking along +x: p_cam = (-y, 1.6 - z, x - 1)."""
    W, H = 22, 8
    f = (W / 2.0) / np.tan(np.radians(35.0))
    f = float(np.float32(f))
    cx, cy = (W - 1) / 2.0, (H - 1) / 2.0
    p = np.array([6.0, 0.5, 1.0])
    h = float(np.float32(1.6))                  # camera height as the fp32 rig stores it in t
    Xc, Yc, Zc = -p[1], h - p[2], p[0] - 1.0
    u = f * Xc / Zc + cx
    v = f * Yc / Zc + cy
    # L = u + 2 v
    dK = np.zeros((3, 3))
    dK[0] = [Xc / Zc, Yc / Zc, 1.0]                    # du/dK_0j
    dK[1] = 2.0 * np.array([Xc / Zc, Yc / Zc, 1.0])     # 2 dv/dK_1j
    dK[2] = -(u + 2.0 * v) * np.array([Xc / Zc, Yc / Zc, 1.0])
    dpc = np.array([f / Zc, 2.0 * f / Zc, -(f * Xc + 2.0 * f * Yc) / Zc ** 2])   # dL/dp_cam
    return {"K": dK, "R": np.outer(dpc, p), "t": dpc, "u": u, "v": v}


def test_golden_single_camera():
    F, K, R, t, rng6, G = golden_setup()
    r = svt.oracle_forward(F, K, R, t, rng6, 1, 1, 1)
    e = golden_expected()
    assert r["counts"][0, 0, 0, 0] == 1
    assert abs(r["out"][0, 0, 0, 0] - e["u"]) < 1e-9 and abs(r["out"][0, 1, 0, 0] - e["v"]) < 1e-9
    got = cg.oracle_camera_backward(G, F, K, R, t, rng6, 1, 1, 1)
    for name in ("K", "R", "t"):
        assert np.abs(got[name][0, 0] - e[name]).max() <= 1e-6 * max(1.0, np.abs(e[name]).max()), name


def test_two_identical_cameras_share_the_gradient():
    F, K, R, t, rng6, G = golden_setup(n_cams=2)
    got = cg.oracle_camera_backward(G, F, K, R, t, rng6, 1, 1, 1)
    e = golden_expected()
    for name in ("K", "R", "t"):
        for n in range(2):
            assert np.abs(got[name][0, n] - 0.5 * e[name]).max() <= 1e-6 * max(1.0, np.abs(e[name]).max()), name


@pytest.mark.parametrize("seed,pitch", [(3, 0.0), (4, 8.0), (5, -10.0)])
def test_homogeneity(seed, pitch):
    F, K, R, t, rng6, X, Y, Z, G = small_case(seed, pitch=pitch, X=16, Y=16, Z=4)
    got = cg.oracle_camera_backward(G, F, K, R, t, rng6, X, Y, Z)
    sK = np.einsum("bnij,bnij->bn", K, got["K"])
    sRt = np.einsum("bnij,bnij->bn", R, got["R"]) + np.einsum("bni,bni->bn", t, got["t"])
    scale = np.abs(got["K"]).max() * np.abs(K).max()
    assert np.abs(got["K"]).max() > 0
    assert np.abs(sK).max() <= 1e-9 * scale
    assert np.abs(sRt).max() <= 1e-9 * max(1.0, np.abs(got["R"]).max() + np.abs(got["t"]).max())


def test_constant_features_give_zero():
    F, K, R, t, rng6, X, Y, Z, G = small_case(6)
    F[:] = 1.75
    got = cg.oracle_camera_backward(G, F, K, R, t, rng6, X, Y, Z)
    for name in ("K", "R", "t"):
        assert np.abs(got[name]).max() <= 1e-12


def test_rows_restriction_is_exact_for_zero_rows():
    F, K, R, t, rng6, X, Y, Z, G = small_case(7)
    rows = np.array([0, 5, 11])
    G2 = np.zeros_like(G)
    G2[:, :, rows] = G[:, :, rows]
    a = cg.oracle_camera_backward(G2, F, K, R, t, rng6, X, Y, Z)
    b = cg.oracle_camera_backward(G2, F, K, R, t, rng6, X, Y, Z, rows=rows)
    for name in ("K", "R", "t"):
        assert np.abs(a[name] - b[name]).max() <= 1e-12 * max(1.0, np.abs(a[name]).max())


# ---- planted mistakes

_orig_proj = cg.projection_gradient
_orig_pix = cg.pixel_gradients
_orig_uvd = cg.sample_uv_derivatives
_orig_all = cg.oracle_camera_backward


def _proj_no_perspective(lu, lv, d, u, v, mask, grid):
    gP = _orig_proj(lu, lv, d, u, v, mask, grid)
    gP[:, 2] = 0.0
    return gP


def _proj_wrong_sign(lu, lv, d, u, v, mask, grid):
    gP = _orig_proj(lu, lv, d, u, v, mask, grid)
    gP[:, 2] *= -1.0
    return gP


def _pix_no_count(grad_out_b, Fb, u, v, mask, rows):
    su, sv = _orig_uvd(Fb, u, v, mask)
    gc = grad_out_b[:, rows]
    return np.einsum("ncryz,cry->nryz", su, gc) * mask, np.einsum("ncryz,cry->nryz", sv, gc) * mask


def _uv_swapped(Fb, u, v, m):
    du, dv = _orig_uvd(Fb, u, v, m)
    return dv, du


def _all_K_not_transposed(grad_out, F, K, R, t, rng6, X, Y, Z, rows=None):
    r = _orig_all(grad_out, F, K, R, t, rng6, X, Y, Z, rows)
    M = np.concatenate([np.asarray(R, np.float64), np.asarray(t, np.float64)[..., None]], axis=-1)
    r["K"] = np.einsum("bnij,bnjk->bnik", r["P"][..., :3], M[..., :3]) + np.einsum("bni,bnk->bnik", r["P"][..., 3],
                                                                                     M[..., 3])
    return r


def _all_RT_not_transposed(grad_out, F, K, R, t, rng6, X, Y, Z, rows=None):
    r = _orig_all(grad_out, F, K, R, t, rng6, X, Y, Z, rows)
    gM = np.einsum("bnik,bnkj->bnij", np.asarray(K, np.float64), r["P"])
    r["R"], r["t"] = gM[..., :3], gM[..., 3]
    return r


def _pins_pass():
    try:
        test_golden_single_camera()
        test_two_identical_cameras_share_the_gradient()
        test_homogeneity(4, 8.0)
        _fd_pin(1, 0.0)
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("name,attr,fn", [
    ("perspective term dropped", "projection_gradient", _proj_no_perspective),
    ("perspective term with the wrong sign", "projection_gradient", _proj_wrong_sign),
    ("valid-camera count left out", "pixel_gradients", _pix_no_count),
    ("d/du and d/dv swapped", "sample_uv_derivatives", _uv_swapped),
    ("dL/dK = dL/dP [R | t] without the transpose", "oracle_camera_backward", _all_K_not_transposed),
    ("dL/d[R | t] = K dL/dP without the transpose", "oracle_camera_backward", _all_RT_not_transposed),
])
def test_mutation_is_caught(monkeypatch, name, attr, fn):
    assert _pins_pass(), "pins must pass on the unmodified oracle"
    monkeypatch.setattr(cg, attr, fn)
    assert not _pins_pass(), f"planted mistake not caught: {name}"
