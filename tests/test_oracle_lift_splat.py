"""CPU: pins of the Lift-Splat (push view transform) oracle.

What fixes it independently of oracle.lift_splat:
  * scalar brute force (oracle.brute_force.lss_brute) on tiny rigs;
  * a golden single point: a camera at yaw 0, the principal-point pixel, all
    depth mass in bin k -> the context lands in the cell of ego point
    (r + d_k, 0, h) (camera at radius r along +x, height h), nowhere else;
  * conservation: with a grid that holds every point, the sum over cells is
    the sum over pixels of (sum_d alpha_d) c;
  * order-free sum over cameras (tutorial, "Splat": the pooling is
    permutation invariant);
  * the backward is the adjoint of the forward (bilinear in alpha and c).
Planted mistakes in the depth of a bin, the camera-to-ego transform, the cell
index and the pooling are each caught by these pins (the brute force left out).
"""
import numpy as np
import pytest

import oracle.lift_splat as ls
from oracle import brute_force as bf
from camera_bev_view_amd import workloads as wl

D_MIN, D_STEP = 4.0, 1.0


def softmax_depth(seed, B, N, D, H, W):
    g = np.random.default_rng([seed, 3])
    z = g.standard_normal((B, N, D, H, W))
    e = np.exp(z - z.max(axis=2, keepdims=True))
    return e / e.sum(axis=2, keepdims=True)


def test_brute_force():
    B, N, D, H, W, C = 2, 3, 6, 4, 5, 3
    K, R, t = wl.make_rig(21, B, N, H, W, True)
    dep = softmax_depth(1, B, N, D, H, W)
    ctx = np.random.default_rng(2).standard_normal((B, N, C, H, W))
    rng6 = (-8.0, 8.0, -8.0, 8.0, -5.0, 3.0)
    o = ls.lss_forward(dep, ctx, K, R, t, rng6, 12, 9, D_MIN, D_STEP)["out"]
    assert np.abs(o).sum() > 0
    ob = np.array(bf.lss_brute(dep.tolist(), ctx.tolist(), *(np.asarray(a, np.float64).tolist() for a in (K, R, t)),
                               rng6, 12, 9, D_MIN, D_STEP))
    assert np.abs(o - ob).max() <= 1e-12


def golden_single_point(k):
    """One camera at yaw 0; H, W odd so the principal point is a pixel centre."""
    H, W, C = 9, 23, 4
    K = wl.intrinsics(H, W)[None, None]
    R, t = wl.extrinsics_from_yaw(0.0)
    dep = np.zeros((1, 1, 41, H, W))
    dep[0, 0, k, (H - 1) // 2, (W - 1) // 2] = 1.0
    ctx = np.zeros((1, 1, C, H, W))
    cvec = np.array([1.5, -2.0, 0.25, 3.0])
    ctx[0, 0, :, (H - 1) // 2, (W - 1) // 2] = cvec
    rng6 = (-50.375, 49.625, -50.375, 49.625, -5.0, 3.0)   # the point 3/4 into its cell: floor and round differ
    return dep, ctx, K, R[None, None], t[None, None], rng6, cvec


@pytest.mark.parametrize("k", [0, 7, 40])
def test_golden_single_point(k):
    dep, ctx, K, R, t, rng6, cvec = golden_single_point(k)
    o = ls.lss_forward(dep, ctx, K, R, t, rng6, 200, 200, D_MIN, D_STEP)["out"]
    x = wl.CAM_RADIUS_M + (D_MIN + k * D_STEP)             # straight ahead along +x
    i = int(np.floor((x - rng6[0]) / 0.5))
    j = int(np.floor((0.0 - rng6[2]) / 0.5))
    expect = np.zeros_like(o)
    expect[0, :, i, j] = cvec
    assert np.abs(o - expect).max() <= 1e-12


@pytest.mark.parametrize("k", [0, 9])
def test_golden_off_axis_point(k):
    """The pixel one focal length right of the principal point looks 45 degrees off axis:
    K^-1 [u, v, 1] = (1, 0, 1), so at camera depth d the point is d right and d ahead."""
    H, W, C = 9, 23, 2
    K = np.array([[[[8.0, 0.0, 11.0], [0.0, 8.0, 4.0], [0.0, 0.0, 1.0]]]], np.float32)
    R, t = wl.extrinsics_from_yaw(0.0)
    dep = np.zeros((1, 1, 41, H, W))
    dep[0, 0, k, 4, 19] = 1.0
    ctx = np.zeros((1, 1, C, H, W))
    ctx[0, 0, :, 4, 19] = [2.0, -1.0]
    rng6 = (-50.375, 49.625, -50.375, 49.625, -5.0, 3.0)
    o = ls.lss_forward(dep, ctx, K, R[None, None], t[None, None], rng6, 200, 200, D_MIN, D_STEP)["out"]
    d = D_MIN + k * D_STEP
    i = int(np.floor((wl.CAM_RADIUS_M + d - rng6[0]) / 0.5))   # ego x: camera centre + d ahead
    j = int(np.floor((-d - rng6[2]) / 0.5))                    # ego y: d to the right (camera x = -ego y)
    expect = np.zeros_like(o)
    expect[0, :, i, j] = [2.0, -1.0]
    assert np.abs(o - expect).max() <= 1e-12


def test_conservation_with_a_grid_holding_every_point():
    B, N, D, H, W, C = 1, 6, 41, 8, 22, 5
    K, R, t = wl.make_rig(22, B, N, H, W, False)
    dep = softmax_depth(3, B, N, D, H, W)
    ctx = np.random.default_rng(4).standard_normal((B, N, C, H, W))
    rng6 = (-60.0, 60.0, -60.0, 60.0, -5.0, 3.0)            # every point is within 45 m + 1 m of the origin
    o = ls.lss_forward(dep, ctx, K, R, t, rng6, 48, 40, D_MIN, D_STEP)["out"]
    expect = (dep.sum(axis=2)[:, :, None] * ctx).sum(axis=(1, 3, 4))    # [B, C]
    assert np.abs(o.sum(axis=(2, 3)) - expect).max() <= 1e-10


def test_camera_permutation():
    B, N, D, H, W, C = 1, 6, 10, 6, 14, 3
    K, R, t = wl.make_rig(23, B, N, H, W, False)
    dep = softmax_depth(5, B, N, D, H, W)
    ctx = np.random.default_rng(6).standard_normal((B, N, C, H, W))
    rng6 = (-20.0, 20.0, -20.0, 20.0, -5.0, 3.0)
    a = ls.lss_forward(dep, ctx, K, R, t, rng6, 30, 30, D_MIN, D_STEP)["out"]
    p = [4, 1, 5, 0, 3, 2]
    b = ls.lss_forward(dep[:, p], ctx[:, p], K[:, p], R[:, p], t[:, p], rng6, 30, 30, D_MIN, D_STEP)["out"]
    assert np.abs(a - b).max() <= 1e-12


def test_backward_is_adjoint():
    B, N, D, H, W, C = 2, 4, 9, 5, 12, 3
    K, R, t = wl.make_rig(24, B, N, H, W, True)
    rng6 = (-15.0, 15.0, -15.0, 15.0, -5.0, 3.0)
    g0 = np.random.default_rng(7)
    dep, ctx = g0.standard_normal((B, N, D, H, W)), g0.standard_normal((B, N, C, H, W))
    ddep, dctx = g0.standard_normal((B, N, D, H, W)), g0.standard_normal((B, N, C, H, W))
    g = g0.standard_normal((B, C, 20, 18))
    gd, gc = ls.lss_backward(g, dep, ctx, K, R, t, rng6, 20, 18, D_MIN, D_STEP)
    # the forward is linear in each argument: <g, d/ds fwd(dep + s ddep, ctx)> = <gd, ddep>, likewise for ctx
    lin_d = ls.lss_forward(ddep, ctx, K, R, t, rng6, 20, 18, D_MIN, D_STEP)["out"]
    lin_c = ls.lss_forward(dep, dctx, K, R, t, rng6, 20, 18, D_MIN, D_STEP)["out"]
    assert abs((g * lin_d).sum() - (gd * ddep).sum()) <= 1e-10 * max(1.0, abs((g * lin_d).sum()))
    assert abs((g * lin_c).sum() - (gc * dctx).sum()) <= 1e-10 * max(1.0, abs((g * lin_c).sum()))


# ---- planted mistakes

_orig_depths = ls.depth_values
_orig_frustum = ls.frustum_points
_orig_cells = ls.bev_cells


def _bin_centres(d_min, d_step, D):
    return _orig_depths(d_min, d_step, D) + 0.5 * d_step


def _frustum_R_not_transposed(K, R, t, H, W, depths):
    return _orig_frustum(K, np.swapaxes(np.asarray(R), -1, -2), t, H, W, depths)


def _frustum_plus_t(K, R, t, H, W, depths):
    return _orig_frustum(K, R, -np.asarray(t), H, W, depths)


def _frustum_range_not_depth(K, R, t, H, W, depths):
    # depth read as distance along the ray instead of the camera-frame z
    K = np.asarray(K, np.float64)
    pts = _orig_frustum(K, R, t, H, W, depths)
    origin = _orig_frustum(K, R, t, H, W, np.zeros(1))
    vs, us = np.meshgrid(np.arange(H, dtype=np.float64), np.arange(W, dtype=np.float64), indexing="ij")
    rays = np.einsum("nij,hwj->nhwi", np.linalg.inv(K), np.stack([us, vs, np.ones_like(us)], -1))
    scale = 1.0 / np.linalg.norm(rays, axis=-1)                         # [N, H, W]
    return origin + (pts - origin) * scale[:, None, :, :, None]


def _cells_xy_swapped(points, rng6, X, Y):
    return _orig_cells(points[..., [1, 0, 2]], rng6, X, Y)


def _cells_rounded(points, rng6, X, Y):
    xmin, xmax, ymin, ymax = (float(r) for r in rng6[:4])
    i = np.round((points[..., 0] - xmin) / ((xmax - xmin) / X))
    j = np.round((points[..., 1] - ymin) / ((ymax - ymin) / Y))
    inside = (i >= 0) & (i < X) & (j >= 0) & (j < Y)
    return np.where(inside, i, 0).astype(np.int64), np.where(inside, j, 0).astype(np.int64), inside


def _pins_pass():
    try:
        for k in (0, 7, 40):
            test_golden_single_point(k)
        for k in (0, 9):
            test_golden_off_axis_point(k)
        test_conservation_with_a_grid_holding_every_point()
        test_camera_permutation()
        test_backward_is_adjoint()
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("name,attr,fn", [
    ("bins at their centres", "depth_values", _bin_centres),
    ("R not transposed", "frustum_points", _frustum_R_not_transposed),
    ("translation added", "frustum_points", _frustum_plus_t),
    ("depth as distance along the ray", "frustum_points", _frustum_range_not_depth),
    ("x and y swapped in the cell index", "bev_cells", _cells_xy_swapped),
    ("cell index rounded, not floored", "bev_cells", _cells_rounded),
])
def test_mutation_is_caught(monkeypatch, name, attr, fn):
    assert _pins_pass(), "pins must pass on the unmodified oracle"
    monkeypatch.setattr(ls, attr, fn)
    assert not _pins_pass(), f"planted mistake not caught: {name}"


def test_points_in_different_cells_add_up():
    dep, ctx, K, R, t, rng6, cvec = golden_single_point(3)
    dep[0, 0, 5, 4, 11] = 1.0                                # a second point in another cell
    a = ls.lss_forward(dep, ctx, K, R, t, rng6, 200, 200, D_MIN, D_STEP)["out"]
    assert np.isclose(a.sum(), 2 * cvec.sum())               # two points, each carrying c: summed, not averaged


def test_near_cell_edge_pins_distances_and_units():
    """Points placed at known metric distances from a cell edge: a 2 m cell grid over [-10, 10) gives
    edges at every even coordinate; eps is in metres, on both axes and at the grid's outer edges."""
    rng6 = (-10.0, 10.0, -10.0, 10.0, -5.0, 3.0)
    X = Y = 10                                      # 2 m cells
    eps = ls.EDGE_EPS_M
    centre = np.array([1.0, -3.0, 0.0])             # a cell centre: 1 m from every edge
    cases = [
        ((centre[0], centre[1]), False),
        ((2.0 + 0.5 * eps, centre[1]), True),       # just inside eps of the x = 2 edge
        ((2.0 - 0.5 * eps, centre[1]), True),       # either side of it
        ((2.0 + 4.0 * eps, centre[1]), False),      # just outside eps
        ((centre[0], -4.0 + 0.5 * eps), True),      # the y axis
        ((centre[0], -4.0 + 4.0 * eps), False),
        ((-10.0 + 0.5 * eps, centre[1]), True),     # the grid's outer edges
        ((10.0 - 0.5 * eps, centre[1]), True),
        ((centre[0], 10.0 - 4.0 * eps), False),
    ]
    pts = np.array([[x, y, 0.0] for (x, y), _ in cases])
    want = np.array([w for _, w in cases])
    assert np.array_equal(ls.near_cell_edge(pts, rng6, X, Y), want)
    # a wider eps in metres flags a point 0.1 m from an edge of a 2 m cell, a narrower one does not
    p = np.array([[2.1, centre[1], 0.0]])
    assert ls.near_cell_edge(p, rng6, X, Y, eps=0.15)[0]
    assert not ls.near_cell_edge(p, rng6, X, Y, eps=0.05)[0]
    # unequal cells: 1 m along x, 4 m along y; a point 0.3 m off a y edge is flagged only for eps > 0.3
    p = np.array([[0.5, 2.3, 0.0]])                 # x: a 1 m cell's centre; y: 0.3 m above the y = 2 edge
    assert ls.near_cell_edge(p, rng6, 20, 5, eps=0.31)[0]
    assert not ls.near_cell_edge(p, rng6, 20, 5, eps=0.29)[0]
