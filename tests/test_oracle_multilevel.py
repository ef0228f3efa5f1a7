"""CPU: pins of the multi-level (feature-pyramid) oracle.

What fixes the multi-level operator independently of oracle.multilevel:
  * with one level it is the single-level operator (itself pinned elsewhere);
  * scalar brute force (oracle.brute_force.cell_value_levels) on tiny grids;
  * constant maps (a different constant per level) give the mean of the level
    constants times the number of bins with a valid camera -- this fixes the
    1/L level mean and the border rule at the edges of coarse levels;
  * a ramp along x written in level-0 pixel units at every level
    (F_l[x] = a + b (r_l x + (r_l - 1)/2), the level-0 coordinate of the
    level-l pixel centre) samples to a + b u at every level for points away
    from the borders -- this fixes the level coordinate mapping;
  * the backward is the adjoint of the forward.
Mutations of the level mapping, the level mean and the border rule are then
planted to check that these pins catch each.
"""
import numpy as np
import pytest

import oracle
import oracle.multilevel as ml
from oracle import brute_force as bf
from camera_bev_view_amd import workloads as wl

RNG20 = (-20.0, 20.0, -20.0, 20.0, -5.0, 3.0)
SHAPES = [(16, 44), (8, 22), (4, 11)]


def pyramid(seed, B, N, C, shapes):
    g = np.random.default_rng([seed, 7])
    return [g.standard_normal((B, N, C, H, W)) for (H, W) in shapes]


def test_level_ratios():
    assert ml.level_ratios(SHAPES) == [1, 2, 4]
    with pytest.raises(ValueError):
        ml.level_ratios([(16, 44), (8, 21)])
    with pytest.raises(ValueError):
        ml.level_ratios([(16, 44), (8, 11)])


def test_one_level_is_the_single_level_operator():
    inp = wl.random_case(3, 2, 6, 5, 8, 22, 7, 9, 4, rng6=RNG20)
    a = ml.oracle_forward_levels([inp.F], inp.K, inp.R, inp.t, inp.rng6, 7, 9, 4)
    b = oracle.oracle_forward(inp.F, inp.K, inp.R, inp.t, inp.rng6, 7, 9, 4)
    assert np.array_equal(a["counts"], b["counts"])
    assert np.abs(a["out"] - b["out"]).max() <= 1e-12
    ga = ml.oracle_backward_levels(inp.grad_out, inp.K, inp.R, inp.t, inp.rng6, 7, 9, 4, [(8, 22)])[0]
    gb = oracle.oracle_backward(inp.grad_out, inp.K, inp.R, inp.t, inp.rng6, 7, 9, 4, 8, 22)
    assert np.abs(ga - gb).max() <= 1e-12


def test_brute_force_three_levels():
    F = pyramid(1, 1, 6, 3, SHAPES)
    K, R, t = wl.make_rig(77, 1, 6, 16, 44, False)
    X, Y, Z = 5, 6, 4
    o = ml.oracle_forward_levels(F, K, R, t, RNG20, X, Y, Z)
    assert (o["counts"] > 0).mean() > 0.3
    lists = [f.tolist() for f in F]
    Kl, Rl, tl = (np.asarray(a, np.float64).tolist() for a in (K, R, t))
    for i in range(X):
        for j in range(Y):
            vals, cs = bf.cell_value_levels(lists, Kl, Rl, tl, RNG20, X, Y, Z, 0, i, j)
            assert list(o["counts"][0, i, j]) == cs
            assert np.abs(np.array(vals) - o["out"][0, :, i, j]).max() <= 1e-12


def test_constant_levels():
    consts = [1.25, -0.5, 3.0]
    F = [np.full((1, 6, 2, H, W), c) for (H, W), c in zip(SHAPES, consts)]
    K, R, t = wl.make_rig(5, 1, 6, 16, 44, False)
    o = ml.oracle_forward_levels(F, K, R, t, RNG20, 9, 11, 6)
    nz = (o["counts"] > 0).sum(axis=-1)                     # [B, X, Y]
    assert nz.max() > 0
    expect = np.mean(consts) * nz
    assert np.abs(o["out"] - expect[:, None]).max() <= 1e-12


def ramp_scene():
    """One camera at yaw 0 looking along +x; a BEV patch 10-20 m ahead, 2 m either
    side, so every valid sample is at least 4 level-0 pixels from the left and
    right borders (the ramp runs along x)."""
    K = wl.intrinsics(16, 44)[None, None]
    R, t = wl.extrinsics_from_yaw(0.0)
    return K, R[None, None], t[None, None], (10.0, 20.0, -2.0, 2.0, -1.0, 3.0)


def test_ramp_fixes_level_coordinates():
    a, b = 0.75, -0.125
    F = []
    for (H, W) in SHAPES:
        r = 16 // H
        x0 = r * np.arange(W) + (r - 1) / 2.0
        F.append(np.broadcast_to(a + b * x0, (1, 1, 1, H, W)).copy())
    K, R, t, rng = ramp_scene()
    X, Y, Z = 6, 5, 4
    o = ml.oracle_forward_levels(F, K, R, t, rng, X, Y, Z)
    grid = oracle.voxel_grid(rng, X, Y, Z)
    d, u, v = oracle.project(grid, K[0], R[0], t[0])
    mask = oracle.in_view_mask(d, u, v, 16, 44)
    assert mask.any()
    assert u[mask].min() > 4 and u[mask].max() < 39
    expect = np.where(mask, a + b * u, 0.0)[0].sum(axis=-1)   # one camera: its sample is the mean
    assert np.abs(o["out"][0, 0] - expect).max() <= 1e-12


def test_backward_is_adjoint():
    K, R, t = wl.make_rig(9, 2, 6, 16, 44, True)
    X, Y, Z = 6, 7, 5
    f = pyramid(2, 2, 6, 3, SHAPES)
    g = np.random.default_rng(3).standard_normal((2, 3, X, Y))
    fwd = ml.oracle_forward_levels(f, K, R, t, RNG20, X, Y, Z)["out"]
    grads = ml.oracle_backward_levels(g, K, R, t, RNG20, X, Y, Z, SHAPES)
    lhs = float((g * fwd).sum())
    rhs = float(sum((gl * fl).sum() for gl, fl in zip(grads, f)))
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs))


# ---- planted mistakes: each must fail at least one of the pins above (brute force left out)

def _coords_no_half_pixel(u, v, r, H, W):
    return np.clip(u / r, 0.0, W - 1.0), np.clip(v / r, 0.0, H - 1.0)


def _coords_wrong_sign(u, v, r, H, W):
    return np.clip((u - 0.5) / r + 0.5, 0.0, W - 1.0), np.clip((v - 0.5) / r + 0.5, 0.0, H - 1.0)


def _sum_over_levels(levels, b, u, v, mask, ratios):
    return _orig_sample(levels, b, u, v, mask, ratios) * len(levels)


def _zero_padding(levels, b, u, v, mask, ratios):
    out = None
    for F, r in zip(levels, ratios):
        H, W = F.shape[-2:]
        ul = (np.where(mask, u, 0.0) + 0.5) / r - 0.5
        vl = (np.where(mask, v, 0.0) + 0.5) / r - 0.5
        inside = mask & (ul >= 0) & (ul <= W - 1) & (vl >= 0) & (vl <= H - 1)
        s = oracle.bilinear_sample(np.asarray(F[b], np.float64), ul, vl, inside)
        out = s if out is None else out + s
    return out / len(levels)


_orig_coords = ml.level_coords
_orig_sample = ml.multilevel_sample


def _pins_pass():
    try:
        test_constant_levels()
        test_ramp_fixes_level_coordinates()
        test_backward_is_adjoint()
        test_one_level_is_the_single_level_operator()
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("name,attr,fn", [
    ("no half-pixel offset in the level mapping", "level_coords", _coords_no_half_pixel),
    ("half-pixel offset with the wrong sign", "level_coords", _coords_wrong_sign),
    ("levels summed, not averaged", "multilevel_sample", _sum_over_levels),
    ("zero padding instead of the border rule", "multilevel_sample", _zero_padding),
])
def test_mutation_is_caught(monkeypatch, name, attr, fn):
    assert _pins_pass(), "pins must pass on the unmodified oracle"
    monkeypatch.setattr(ml, attr, fn)
    assert not _pins_pass(), f"planted mistake not caught: {name}"
