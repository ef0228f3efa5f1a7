"""CPU: pins of the temporal fused view transform oracle (oracle.temporal).

What fixes it independently of oracle.temporal:
  * scalar brute force (oracle.brute_force.align_brute);
  * the identity motion returns the previous map unchanged;
  * a translation by three cells along x shifts the map by three rows (zeros
    where the previous grid did not reach); half a cell along y gives the mean
    of neighbouring columns;
  * a +90 degree turn about the centre of a square, centred grid equals
    numpy's rot90 of the previous map (fixes the direction of A and the
    row / column roles);
  * the adjoint identity <align(p), g> = <p, align^T(g)>;
  * constant maps give the constant inside the covered box and 0 outside;
  * the first C channels are the Sampling-VT oracle's, forward and backward.
Planted mistakes are each caught by these pins (the brute force left out).
"""
import numpy as np
import pytest

import oracle.sampling_vt as svt
import oracle.temporal as tp
from oracle import brute_force as bf
from camera_bev_view_amd import workloads as wl

RNG = (-8.0, 8.0, -6.0, 6.0, -2.0, 2.0)


def rigid(theta_deg, tx, ty, B=1):
    th = np.radians(theta_deg)
    A = np.array([[np.cos(th), -np.sin(th), tx], [np.sin(th), np.cos(th), ty]])
    return np.repeat(A[None], B, axis=0)


def prev_map(seed, B=1, Cp=3, X=16, Y=12):
    return np.random.default_rng(seed).standard_normal((B, Cp, X, Y))


def test_brute_force():
    for seed, (th, tx, ty) in enumerate([(7.0, 0.6, -0.3), (-20.0, 1.7, 2.2), (180.0, 0.0, 0.0)]):
        P = prev_map(seed, B=2)
        A = np.stack([rigid(th, tx, ty)[0], rigid(-th / 2, -tx, ty)[0]])
        got = tp.align_prev_bev(P, A, RNG)["aligned"]
        for b in range(2):
            for c in range(P.shape[1]):
                for i in range(P.shape[2]):
                    for j in range(P.shape[3]):
                        ref = bf.align_brute(P[b].tolist(), A[b].tolist(), RNG, P.shape[2], P.shape[3], c, i, j)
                        assert abs(got[b, c, i, j] - ref) <= 1e-12


def test_identity():
    P = prev_map(1)
    r = tp.align_prev_bev(P, rigid(0, 0, 0), RNG)
    assert np.array_equal(r["aligned"], P) and r["inside"].all()


def test_integer_shift_along_x():
    P = prev_map(2)
    X = P.shape[2]
    dx = (RNG[1] - RNG[0]) / X
    got = tp.align_prev_bev(P, rigid(0, 3 * dx, 0), RNG)["aligned"]
    assert np.allclose(got[:, :, :X - 3], P[:, :, 3:], atol=1e-12)
    assert not got[:, :, X - 3:].any()


def test_half_cell_shift_along_y():
    P = prev_map(3)
    Y = P.shape[3]
    dy = (RNG[3] - RNG[2]) / Y
    got = tp.align_prev_bev(P, rigid(0, 0, 0.5 * dy), RNG)["aligned"]
    assert np.allclose(got[..., :Y - 1], 0.5 * (P[..., :Y - 1] + P[..., 1:]), atol=1e-12)
    assert not got[..., Y - 1].any()


def test_quarter_turn_is_rot90():
    P = prev_map(4, X=10, Y=10)
    sq = (-5.0, 5.0, -5.0, 5.0, -1.0, 1.0)
    got = tp.align_prev_bev(P, rigid(90.0, 0, 0), sq)["aligned"]
    assert np.allclose(got, np.rot90(P, k=-1, axes=(2, 3)), atol=1e-12)


def test_adjoint_identity():
    P = prev_map(5, B=2)
    G = np.random.default_rng(6).standard_normal(P.shape)
    A = np.stack([rigid(12.0, 0.8, -1.1)[0], rigid(-33.0, -2.0, 0.4)[0]])
    lhs = (tp.align_prev_bev(P, A, RNG)["aligned"] * G).sum()
    rhs = (P * tp.align_adjoint(G, A, RNG)).sum()
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs))


def test_constant_map():
    P = np.full((1, 2, 16, 12), 1.5)
    r = tp.align_prev_bev(P, rigid(25.0, 1.2, -0.7), RNG)
    assert r["inside"].any() and (~r["inside"]).any()
    assert np.allclose(r["aligned"], 1.5 * r["inside"][:, None], atol=1e-12)


def test_current_channels_are_the_sampling_vt():
    inp = wl.random_case(7, 1, 6, 4, 8, 22, 12, 10, 3, rng6=(-20.0, 20.0, -20.0, 20.0, -4.0, 3.0))
    P = prev_map(8, Cp=2, X=12, Y=10)
    A = rigid(5.0, 0.4, 0.2)
    r = tp.temporal_forward(inp.F, inp.K, inp.R, inp.t, inp.rng6, 12, 10, 3, P, A)
    ref = svt.oracle_forward(inp.F, inp.K, inp.R, inp.t, inp.rng6, 12, 10, 3)
    assert r["out"].shape == (1, 6, 12, 10)
    assert np.array_equal(r["out"][:, :4], ref["out"])
    assert np.array_equal(r["out"][:, 4:], tp.align_prev_bev(P, A, inp.rng6)["aligned"])
    G = np.random.default_rng(9).standard_normal((1, 6, 12, 10))
    gF, gP = tp.temporal_backward(G, inp.K, inp.R, inp.t, inp.rng6, 12, 10, 3, 8, 22, 4, A)
    assert np.array_equal(gF, svt.oracle_backward(G[:, :4], inp.K, inp.R, inp.t, inp.rng6, 12, 10, 3, 8, 22))
    assert np.array_equal(gP, tp.align_adjoint(G[:, 4:], A, inp.rng6))


# ---- planted mistakes

_orig_src = tp.source_indices
_orig_align = tp.align_prev_bev


def _src_transposed(A, rng6, X, Y):
    return _orig_src(np.asarray(A)[:, [1, 0, 2]], rng6, X, Y)


def _src_no_half_cell(A, rng6, X, Y):
    si, sj = _orig_src(A, rng6, X, Y)
    return si + 0.5, sj + 0.5


def _src_inverse_rotation(A, rng6, X, Y):
    A = np.array(A, np.float64)
    A[0, 1], A[1, 0] = A[1, 0], A[0, 1]
    return _orig_src(A, rng6, X, Y)


def _align_clamped_border(prev, A, rng6):
    prev = np.asarray(prev, np.float64)
    B, Cp, X, Y = prev.shape
    out = np.zeros_like(prev)
    for b in range(B):
        si, sj = _orig_src(A[b], rng6, X, Y)
        si, sj = np.clip(si, 0, X - 1), np.clip(sj, 0, Y - 1)
        for (ii, jj, w) in svt.bilinear_taps(sj, si, np.ones_like(si, bool), X, Y):
            out[b] += prev[b][:, ii, jj] * w[None]
    return {"aligned": out, "inside": np.ones((B, X, Y), bool), "near_border": np.zeros((B, X, Y), bool)}


def _pins_pass():
    try:
        test_identity()
        test_integer_shift_along_x()
        test_half_cell_shift_along_y()
        test_quarter_turn_is_rot90()
        test_constant_map()
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("name,attr,fn", [
    ("x and y of the motion swapped", "source_indices", _src_transposed),
    ("no half-cell offset", "source_indices", _src_no_half_cell),
    ("rotation applied the other way", "source_indices", _src_inverse_rotation),
    ("border replication instead of zeros", "align_prev_bev", _align_clamped_border),
])
def test_mutation_is_caught(monkeypatch, name, attr, fn):
    assert _pins_pass(), "pins must pass on the unmodified oracle"
    monkeypatch.setattr(tp, attr, fn)
    assert not _pins_pass(), f"planted mistake not caught: {name}"


def test_near_border_pins_distances():
    """A pure shift along x by s cells moves every source index to i + s; the box's edges are at
    0 and X - 1, so a shift of -(1 - d) puts column 1 at distance d from the lower edge and a
    shift of +(1 - d) puts column X - 2 at distance d from the upper edge."""
    rng6 = (-10.0, 10.0, -8.0, 8.0, -5.0, 3.0)
    X, Y = 10, 8                                       # 2 m cells along both axes
    prev = np.zeros((1, 1, X, Y))
    e = svt.EDGE_EPS_PX
    for d, flagged in ((0.5 * e, True), (4.0 * e, False)):
        for sign in (-1.0, 1.0):
            s = sign * (1.0 - d)                      # cells
            A = np.array([[[1.0, 0.0, 2.0 * s], [0.0, 1.0, 0.0]]])
            nb = tp.align_prev_bev(prev, A, rng6)["near_border"][0]
            row = 1 if sign < 0 else X - 2
            inner = nb[:, 1:Y - 1]                    # columns whose source is off the y edges
            assert bool(inner[row].all()) == flagged, (d, sign)
            # the other rows are at least one cell inside or outside the box: never flagged there
            others = np.ones(X, bool)
            others[row] = False
            assert not inner[others].any(), (d, sign)
            # columns 0 and Y - 1 sit exactly on the y edges: flagged wherever the source row is in the box
            si = np.arange(X) + s
            in_box = (si > -e) & (si < X - 1 + e)
            assert np.array_equal(nb[:, 0], in_box) and np.array_equal(nb[:, Y - 1], in_box), (d, sign)
    # the same along y, with the box's edges at 0 and Y - 1
    A = np.array([[[1.0, 0.0, 0.0], [0.0, 1.0, 2.0 * (1.0 - 0.5 * e)]]])
    nb = tp.align_prev_bev(prev, A, rng6)["near_border"][0]
    assert nb[1:X - 1, Y - 2].all() and not nb[1:X - 1, :Y - 2].any() and not nb[1:X - 1, Y - 1].any()
    # sources far outside the box are never flagged, however close to a grid line
    A = np.array([[[1.0, 0.0, 2.0 * 20.0], [0.0, 1.0, 0.0]]])
    assert not tp.align_prev_bev(prev, A, rng6)["near_border"].any()
