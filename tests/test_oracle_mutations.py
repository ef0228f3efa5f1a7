"""CPU: plausible mistakes planted in the oracle are caught by the pins.

Each mutation replaces one oracle stage with a subtly wrong version (a
dropped term, a wrong sign or index, a transposed operand, a different
reading of an open point).  The brute-force pin is left out on purpose: a
misreading shared by both scalar and numpy code would slip past it, so the
closed forms, invariants and library cross-checks must catch each one alone.
"""
import numpy as np
import pytest

import oracle_pins as P
import oracle.sampling_vt as ovt
from camera_bev_view_amd import workloads as wl

_orig = {name: getattr(ovt, name) for name in
         ("valid_camera_mean", "height_sum", "bilinear_taps", "in_view_mask", "project", "voxel_grid")}


def _mean_over_all_cameras(samples, mask):
    cnt = mask.sum(axis=0)
    return samples.sum(axis=0) / mask.shape[0], cnt


def _mean_over_height(m):
    return m.mean(axis=-1)


def _swapped_fractions(u, v, mask, H, W):
    taps = _orig["bilinear_taps"](u, v, mask, H, W)
    # weights of the x-neighbours taken from the v fraction and vice versa
    (y0, x0, w00), (_, x1, w01), (y1, _, w10), (_, _, w11) = taps
    return [(y0, x0, w00), (y0, x1, w10), (y1, x0, w01), (y1, x1, w11)]


def _no_depth_test(d, u, v, H, W):
    with np.errstate(invalid="ignore"):
        return (u >= 0) & (u <= W - 1) & (v >= 0) & (v <= H - 1)


def _open_pixel_box(d, u, v, H, W):
    with np.errstate(invalid="ignore"):
        return (d > 0) & (u >= 0) & (u <= W) & (v >= 0) & (v <= H)


def _project_transposed_R(points, K, R, t):
    return _orig["project"](points, K, np.swapaxes(np.asarray(R), -1, -2), t)


def _project_minus_t(points, K, R, t):
    return _orig["project"](points, K, R, -np.asarray(t))


def _voxel_corners(rng6, X, Y, Z, rows=None):
    g = _orig["voxel_grid"](rng6, X, Y, Z, rows)
    xmin, xmax, ymin, ymax, zmin, zmax = rng6
    return g - 0.5 * np.array([(xmax - xmin) / X, (ymax - ymin) / Y, (zmax - zmin) / Z])


def _taps_uv_swapped(u, v, mask, H, W):
    # samples F[x, y] instead of F[y, x] (only in range when both fit; clipped otherwise)
    taps = _orig["bilinear_taps"](u, v, mask, H, W)
    return [(np.clip(xx, 0, H - 1), np.clip(yy, 0, W - 1), w) for (yy, xx, w) in taps]


MUTATIONS = {
    "mean_divides_by_N": ("valid_camera_mean", _mean_over_all_cameras),
    "height_mean_not_sum": ("height_sum", _mean_over_height),
    "bilinear_fractions_swapped": ("bilinear_taps", _swapped_fractions),
    "depth_test_dropped": ("in_view_mask", _no_depth_test),
    "in_view_box_0_to_W": ("in_view_mask", _open_pixel_box),
    "R_transposed": ("project", _project_transposed_R),
    "t_sign_flipped": ("project", _project_minus_t),
    "voxel_corner_not_centre": ("voxel_grid", _voxel_corners),
    "image_axes_swapped": ("bilinear_taps", _taps_uv_swapped),
}


def _pins():
    small = P.small_case(0)
    tiny = wl.make_inputs("tiny", with_grad=True)
    return [
        ("constant", lambda: P.pin_constant_features(small)),
        ("zero_valid", lambda: P.pin_zero_valid(small)),
        ("behind", P.pin_behind_single_camera),
        ("closed_forms", P.pin_closed_forms),
        ("symmetry", P.pin_rig_symmetry),
        ("library", P.pin_library_bilinear),
        ("adjoint", lambda: P.pin_adjoint(tiny)),
    ]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(monkeypatch, name):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(ovt, attr, fn)
    caught = []
    for pin_name, pin in _pins():
        try:
            pin()
        except (AssertionError, IndexError, ValueError):
            caught.append(pin_name)
    assert caught, f"no pin caught mutation {name}"


_orig_bwd = ovt.oracle_backward


def test_backward_mutation_dropped_count_is_caught(monkeypatch):
    """A backward that forgets the 1/count of the valid mean breaks the adjoint identity."""
    monkeypatch.setattr(ovt, "valid_mean_adjoint_scale", lambda mask: mask.astype(np.float64))
    with pytest.raises(AssertionError):
        P.pin_adjoint(P.small_case(0))


def test_backward_mutation_transposed_tap_is_caught(monkeypatch):
    """A backward that scatters onto (x, y) instead of (y, x) breaks the Jacobian pin."""
    real_taps = ovt.bilinear_taps

    def bad(grad_out, K, R, t, rng6, X, Y, Z, H, W):
        ovt.bilinear_taps = lambda u, v, m, H_, W_: [(np.minimum(xx, H_ - 1), np.minimum(yy, W_ - 1), w)
                                                     for (yy, xx, w) in real_taps(u, v, m, H_, W_)]
        try:
            return _orig_bwd(grad_out, K, R, t, rng6, X, Y, Z, H, W)
        finally:
            ovt.bilinear_taps = real_taps

    monkeypatch.setattr(ovt, "oracle_backward", bad)
    with pytest.raises(AssertionError):
        P.pin_jacobian()
