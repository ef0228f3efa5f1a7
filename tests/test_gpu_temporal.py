"""GPU: the temporal fused view transform (fbev_forward_temporal /
fbev_backward_temporal) against the fp64 oracle (oracle.temporal).

Parity rules:
  * channels [0, C) (the current frame's Sampling-VT) as for fbev_forward:
    within 1e-4 + 1e-5 |ref| except cells with a sample within 1e-4 px of an
    image edge;
  * channels [C, C + Cp) (the aligned previous map) within 1e-4 + 1e-5 |ref|
    except cells whose source lies within 1e-4 cells of the previous grid's
    border (a rounding flip of the in-box test there changes the value);
  * dL/dF and dL/dprev within 1e-3 relative L2, dL/dprev also element-wise
    within 1e-4 + 1e-5 max|ref| on an upstream gradient zeroed at the
    excluded cells.
Every case prints its label before the GPU work starts.
"""
import numpy as np
import pytest
import torch

import oracle.temporal as tp
from camera_bev_view_amd import ops
from camera_bev_view_amd import workloads as wl
from gpu_helpers import ATOL, BWD_REL_L2, RTOL, rel_l2, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def temporal_parity(ti, label, backward=True, exact=False, on_grid_lines=False):
    """``on_grid_lines``: a motion that maps the current grid onto the previous one (the identity, a quarter
    turn of a square grid), so every border cell's source sits on the box's edge and the exclusion bound
    does not apply; such cases are compared bit for bit inside the border by their test."""
    cur = ti.cur
    B, N, C, H, W = cur.F.shape
    X, Y, Z = cur.X, cur.Y, cur.Z
    Cp = ti.prev.shape[1]
    say(f"[case] temporal {label}: B,N,C={B},{N},{C} Cp={Cp} grid {X}x{Y}x{Z}")
    F, K, R, t = to_device(cur)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    prev, ego = dev(ti.prev), dev(ti.ego)
    out, _ = ops.forward_temporal(F, K, R, t, cur.rng6, X, Y, Z, prev, ego)
    torch.cuda.synchronize()
    ref = tp.temporal_forward(cur.F, cur.K, cur.R, cur.t, cur.rng6, X, Y, Z, ti.prev, ti.ego)
    got = out.cpu().numpy()
    cell_ok = ~ref["near_edge"].any(axis=-1)                       # [B, X, Y]
    border_ok = np.ones_like(cell_ok) if exact else ~ref["near_border"]
    diff = np.abs(got - ref["out"])
    tol = ATOL + RTOL * np.abs(ref["out"])
    bad_cur = (diff[:, :C] > tol[:, :C]) & cell_ok[:, None]
    bad_prev = (diff[:, C:] > tol[:, C:]) & border_ok[:, None]
    say(f"[parity] temporal {label}: current max|d|={diff[:, :C].max(initial=0):.3e} aligned max|d|="
        f"{np.where(border_ok[:, None], diff[:, C:], 0).max(initial=0):.3e} excluded cells "
        f"{int((~cell_ok).sum())} / {int((~border_ok).sum())}")
    # the border exclusion may only drop a handful of cells: at most 4, or 0.1% of a larger grid
    if not on_grid_lines:
        assert int((~border_ok).sum()) <= max(4, (B * X * Y) // 1000), f"{label}: {int((~border_ok).sum())} excluded"
    assert not bad_cur.any(), f"{label}: {int(bad_cur.sum())} current-frame outputs outside tolerance"
    assert not bad_prev.any(), f"{label}: {int(bad_prev.sum())} aligned outputs outside tolerance"
    if not backward:
        return out
    G = np.array(ti.grad_out, np.float32, copy=True)
    G[np.broadcast_to((~border_ok)[:, None], G.shape) & (np.arange(C + Cp) >= C)[None, :, None, None]] = 0.0
    gF, gP = ops.backward_temporal(dev(G), (B, N, H, W, C), K, R, t, cur.rng6, X, Y, Z, Cp, ego)
    torch.cuda.synchronize()
    rF, rP = tp.temporal_backward(G, cur.K, cur.R, cur.t, cur.rng6, X, Y, Z, H, W, C, ti.ego)
    gF = gF.cpu().numpy().transpose(0, 1, 4, 2, 3)
    gP = gP.cpu().numpy()
    eF, eP = rel_l2(gF, rF), rel_l2(gP, rP)
    say(f"[parity] temporal {label}: backward rel L2 features {eF:.3e} previous map {eP:.3e}")
    if np.linalg.norm(rF) > 0:
        assert eF <= BWD_REL_L2, f"{label}: dL/dF rel L2 {eF:.3e}"
    if np.linalg.norm(rP) > 0:
        assert eP <= BWD_REL_L2, f"{label}: dL/dprev rel L2 {eP:.3e}"
    assert np.abs(gP - rP).max(initial=0) <= ATOL + RTOL * np.abs(rP).max(initial=0), f"{label}: dL/dprev element"
    return out


def test_temporal_workload():
    """nuScenes-shaped current frame, a 64-channel previous map, a seeded half-second motion."""
    temporal_parity(wl.make_temporal_inputs("temporal"), "nuScenes-shaped")


TEMPORAL_CASES = [
    # label, B, N, C, H, W, X, Y, Z, Cp, yaw, shift
    ("two samples, ragged grid and chunk tail", 2, 6, 12, 8, 22, 23, 37, 4, 13, None, None),
    ("two samples, one launch per direction", 2, 6, 32, 8, 22, 21, 34, 4, 11, 8.0, (1.5, -0.5)),
    ("one previous channel, strong turn", 1, 6, 8, 8, 22, 30, 30, 3, 1, 35.0, (3.0, -2.0)),
    ("no current channels", 1, 6, 0, 8, 22, 20, 24, 3, 9, 10.0, (1.0, 1.0)),
    ("backwards motion off the grid", 1, 6, 4, 8, 22, 16, 16, 3, 5, -3.0, (-40.0, 0.0)),
    # bf16 features with the resampling fused into the forward's last (16-lane) channel group
    ("bf16 features, fused last group", 1, 6, 64, 16, 44, 40, 36, 6, 7, 12.0, (2.0, 1.0), "bf16"),
    # fp32 with two channel groups (256 + 64): the first launched alone, the last one fused with the resampling
    ("two channel groups, last fused", 1, 6, 320, 8, 22, 19, 41, 4, 6, -9.0, (-1.0, 2.5)),
    # 256 + 4 channels: the last group's 4-lane layout has no fused form, so the resampling runs on its own
    ("two channel groups, separate resampling", 1, 6, 260, 8, 22, 17, 23, 4, 3, 5.0, (0.5, -1.5)),
    # 64 fp32 / 128 bf16 channels (256 bytes a pixel): the bin-run forward's tiles and the resampling in one launch
    ("bin-run forward fused, fp32", 2, 6, 64, 8, 22, 26, 35, 5, 9, -14.0, (1.0, -2.0)),
    ("bin-run forward fused, bf16", 1, 6, 128, 8, 22, 18, 29, 4, 5, 7.0, (-0.5, 1.5), "bf16"),
]


@pytest.mark.parametrize("case", TEMPORAL_CASES, ids=[c[0] for c in TEMPORAL_CASES])
def test_temporal_cases(case):
    label, B, N, C, H, W, X, Y, Z, Cp, yaw, shift = case[:12]
    dtype = case[12] if len(case) > 12 else "f32"
    temporal_parity(wl.random_temporal_case(len(label), B, N, C, H, W, X, Y, Z, Cp, yaw_deg=yaw, shift=shift,
                                            dtype=dtype), label)


def test_identity_and_quarter_turn_are_exact():
    """No motion: the previous map comes back bit for bit inside the box; a quarter turn of a square,
    centred grid is numpy's rot90."""
    sq = (-10.0, 10.0, -10.0, 10.0, -4.0, 3.0)
    ti = wl.random_temporal_case(3, 1, 6, 4, 8, 22, 20, 20, 3, 6, rng6=sq, yaw_deg=0.0, shift=(0.0, 0.0))
    out = temporal_parity(ti, "identity", backward=False, on_grid_lines=True)
    assert np.array_equal(out.cpu().numpy()[:, 4:, 1:-1, 1:-1], ti.prev[:, :, 1:-1, 1:-1])
    ti = wl.random_temporal_case(4, 1, 6, 4, 8, 22, 20, 20, 3, 6, rng6=sq, yaw_deg=90.0, shift=(0.0, 0.0))
    out = temporal_parity(ti, "quarter turn", backward=False, on_grid_lines=True)
    rot = np.rot90(ti.prev, k=-1, axes=(2, 3))
    assert np.abs(out.cpu().numpy()[:, 4:, 1:-1, 1:-1] - rot[:, :, 1:-1, 1:-1]).max() <= 1e-6


def test_no_previous_channels_equals_forward():
    ti = wl.random_temporal_case(5, 1, 6, 16, 8, 22, 24, 24, 4, 0)
    say("[case] temporal Cp = 0")
    F, K, R, t = to_device(ti.cur)
    prev = torch.empty((1, 0, 24, 24), device="cuda")
    ego = torch.from_numpy(ti.ego).cuda()
    a, _ = ops.forward_temporal(F, K, R, t, ti.cur.rng6, 24, 24, 4, prev, ego)
    b, _ = ops.forward(F, K, R, t, ti.cur.rng6, 24, 24, 4)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_backward_deterministic_and_autograd():
    ti = wl.random_temporal_case(6, 1, 6, 8, 8, 22, 28, 28, 3, 10, yaw_deg=12.0, shift=(2.5, 0.5))
    say("[case] temporal determinism and autograd")
    F, K, R, t = to_device(ti.cur)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    prev, ego, g = dev(ti.prev), dev(ti.ego), dev(ti.grad_out)
    shape = tuple(F.shape)
    _, p1 = ops.backward_temporal(g, shape, K, R, t, ti.cur.rng6, 28, 28, 3, 10, ego)
    _, p2 = ops.backward_temporal(g, shape, K, R, t, ti.cur.rng6, 28, 28, 3, 10, ego)
    F.requires_grad_(True)
    prev.requires_grad_(True)
    out = ops.TemporalVT.apply(F, prev, K, R, t, ego, ti.cur.rng6, 28, 28, 3)
    gF, gP = torch.autograd.grad(out, (F, prev), g)
    torch.cuda.synchronize()
    assert torch.equal(p1, p2) and torch.equal(gP, p1)
    assert gF.shape == F.shape
