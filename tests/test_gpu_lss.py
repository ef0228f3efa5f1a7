"""GPU: the Lift-Splat entry points (fbev_lss_forward / fbev_lss_backward)
against the fp64 Lift-Splat oracle.

Parity rules:
  * forward pillar sums within |d| <= 1e-4 + 1e-5 |ref|, except the cells
    within one cell of a point that lies within 1e-9 m of a cell edge (its
    cell is a rounding decision, and either side is correct);
  * dL/ddepth and dL/dcontext within 1e-3 relative L2 overall, and element
    by element within 1e-4 + 1e-5 |ref| away from such points (their pixels
    for dL/dcontext).
Every case prints its label before the GPU work starts.
"""
import numpy as np
import pytest
import torch

import oracle.lift_splat as ls
from camera_bev_view_amd import ops
from camera_bev_view_amd import workloads as wl
from gpu_helpers import ATOL, BWD_REL_L2, RTOL, rel_l2, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def device_inputs(inp):
    """Channels-last depth [B,N,H,W,D] and context [B,N,H,W,C] plus K, R, t on the GPU."""
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return (dev(inp.depth.transpose(0, 1, 3, 4, 2)), dev(inp.context.transpose(0, 1, 3, 4, 2)),
            dev(inp.K), dev(inp.R), dev(inp.t))


def edge_masks(inp):
    """(cells [B,X,Y] to leave out, points [B,N,D,H,W] near an edge, pixels [B,N,H,W] with such a point)."""
    B, N, D, H, W = inp.depth.shape
    X, Y = inp.X, inp.Y
    xmin, xmax, ymin, ymax = inp.rng6[:4]
    cells = np.zeros((B, X, Y), bool)
    near = np.zeros((B, N, D, H, W), bool)
    zs = ls.depth_values(inp.d_min, inp.d_step, D)
    for b in range(B):
        pts = ls.frustum_points(inp.K[b], inp.R[b], inp.t[b], H, W, zs)
        near[b] = ls.near_cell_edge(pts, inp.rng6, X, Y)
        fi = np.floor((pts[..., 0][near[b]] - xmin) / ((xmax - xmin) / X)).astype(np.int64)
        fj = np.floor((pts[..., 1][near[b]] - ymin) / ((ymax - ymin) / Y)).astype(np.int64)
        for di in (-1, 0, 1):
            for dj in (-1, 0, 1):
                i, j = fi + di, fj + dj
                ok = (i >= 0) & (i < X) & (j >= 0) & (j < Y)
                cells[b, i[ok], j[ok]] = True
    return cells, near, near.any(axis=2)


def lss_parity(inp, label, backward=True):
    B, N, D, H, W = inp.depth.shape
    C = inp.context.shape[2]
    say(f"[case] lss {label}: B,N,C,D={B},{N},{C},{D} HxW={H}x{W} X,Y={inp.X},{inp.Y} "
        f"bins {inp.d_min}+k*{inp.d_step}")
    dep, ctx, K, R, t = device_inputs(inp)
    out = ops.lss_forward(dep, ctx, K, R, t, inp.rng6, inp.X, inp.Y, inp.d_min, inp.d_step)
    torch.cuda.synchronize()
    ref = ls.lss_forward(inp.depth, inp.context, inp.K, inp.R, inp.t, inp.rng6, inp.X, inp.Y, inp.d_min,
                         inp.d_step)["out"]
    cells, near, near_pix = edge_masks(inp)
    got = out.cpu().numpy()
    diff = np.abs(got - ref)
    bad = (diff > ATOL + RTOL * np.abs(ref)) & ~cells[:, None]
    say(f"[parity] lss {label}: forward max|d|={diff.max(initial=0):.3e} excluded cells={int(cells.sum())} "
        f"near-edge points={int(near.sum())} nonzero outputs={int((ref != 0).sum())}")
    assert not bad.any(), f"{label}: {int(bad.sum())} outputs outside tolerance, worst {diff[bad].max():.3e}"
    # the exclusion may only drop a handful of cells: at most 9 (one point's neighbourhood), or 0.1% of a larger grid
    assert int(cells.sum()) <= max(9, (B * inp.X * inp.Y) // 1000), f"{label}: {int(cells.sum())} cells excluded"
    if not backward:
        return got, ref
    gd, gc = ops.lss_backward(torch.from_numpy(inp.grad_out).cuda(), dep, ctx, K, R, t, inp.rng6, inp.X, inp.Y,
                              inp.d_min, inp.d_step)
    torch.cuda.synchronize()
    rd, rc = ls.lss_backward(inp.grad_out, inp.depth, inp.context, inp.K, inp.R, inp.t, inp.rng6, inp.X, inp.Y,
                             inp.d_min, inp.d_step)
    gd = gd.cpu().numpy().transpose(0, 1, 4, 2, 3)
    gc = gc.cpu().numpy().transpose(0, 1, 4, 2, 3)
    ed, ec = rel_l2(gd, rd), rel_l2(gc, rc)
    say(f"[parity] lss {label}: backward rel L2 depth {ed:.3e} context {ec:.3e}")
    if np.linalg.norm(rd) > 0:
        assert ed <= BWD_REL_L2
    else:
        assert not gd.any()
    if np.linalg.norm(rc) > 0:
        assert ec <= BWD_REL_L2
    else:
        assert not gc.any()
    bad_d = (np.abs(gd - rd) > ATOL + RTOL * np.abs(rd)) & ~near
    bad_c = (np.abs(gc - rc) > ATOL + RTOL * np.abs(rc)) & ~near_pix[:, :, None]
    assert not bad_d.any(), f"{label}: {int(bad_d.sum())} dL/ddepth elements outside tolerance"
    assert not bad_c.any(), f"{label}: {int(bad_c.sum())} dL/dcontext elements outside tolerance"
    return got, ref


def test_lss_nuscenes_tutorial_sizes():
    """Six cameras, 8 x 22 maps, C = 64, 41 bins over [4, 45) m, 200 x 200 cells of 0.5 m."""
    lss_parity(wl.make_lss_inputs("lss", with_grad=True), "tutorial sizes")


def test_lss_batched():
    lss_parity(wl.make_lss_inputs("lss_batched", with_grad=True), "batched 4 x 16x44")


LSS_CASES = [
    # label, B, N, C, H, W, D, X, Y, rng6, d_min, d_step, pitch
    ("ragged grid, two channel groups, pitch", 2, 6, 80, 6, 10, 13, 37, 29, (-20.0, 20.0, -18.0, 17.0, -5.0, 3.0),
     2.0, 1.5, 8.0),
    ("three channel groups", 1, 4, 130, 4, 6, 9, 23, 21, (-15.0, 15.0, -15.0, 15.0, -5.0, 3.0), 1.0, 1.0, -5.0),
    ("fine depth steps: crossings longer than 64 bins", 1, 6, 16, 4, 12, 300, 40, 40,
     (-20.0, 20.0, -20.0, 20.0, -5.0, 3.0), 4.0, 0.05, 0.0),
    ("one channel, one bin, 1x1 maps", 2, 3, 1, 1, 1, 1, 12, 12, (-10.0, 10.0, -10.0, 10.0, -5.0, 3.0), 5.0, 1.0,
     0.0),
    ("coarse cells, many points per cell", 1, 6, 64, 8, 22, 41, 5, 7, (-50.0, 50.0, -50.0, 50.0, -5.0, 3.0), 4.0,
     1.0, 3.0),
    ("grid far from every point", 1, 6, 8, 4, 8, 10, 16, 16, (500.0, 520.0, 500.0, 520.0, -5.0, 3.0), 4.0, 1.0, 0.0),
]


@pytest.mark.parametrize("case", LSS_CASES, ids=[c[0] for c in LSS_CASES])
def test_lss_cases(case):
    label, B, N, C, H, W, D, X, Y, rng6, d_min, d_step, pitch = case
    inp = wl.random_lss_case(len(label), B, N, C, H, W, D, X, Y, rng6, d_min, d_step, pitch)
    lss_parity(inp, label)


def test_lss_conservation_on_gpu():
    """A grid holding every point: the pillar sums add up to sum over pixels of (sum_k alpha_k) c."""
    inp = wl.random_lss_case(7, 2, 6, 24, 8, 22, 41, 60, 52, (-60.0, 60.0, -60.0, 60.0, -5.0, 3.0))
    say("[case] lss conservation")
    dep, ctx, K, R, t = device_inputs(inp)
    out = ops.lss_forward(dep, ctx, K, R, t, inp.rng6, inp.X, inp.Y, inp.d_min, inp.d_step)
    torch.cuda.synchronize()
    total = out.double().sum(dim=(2, 3)).cpu().numpy()
    expect = (inp.depth.astype(np.float64).sum(axis=2)[:, :, None] * inp.context).sum(axis=(1, 3, 4))
    assert np.abs(total - expect).max() <= 1e-3 * max(1.0, np.abs(expect).max())


def test_lss_forward_is_deterministic():
    inp = wl.make_lss_inputs("lss")
    say("[case] lss determinism")
    dep, ctx, K, R, t = device_inputs(inp)
    a = ops.lss_forward(dep, ctx, K, R, t, inp.rng6, inp.X, inp.Y, inp.d_min, inp.d_step)
    b = ops.lss_forward(dep, ctx, K, R, t, inp.rng6, inp.X, inp.Y, inp.d_min, inp.d_step)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_lss_overwrites_outputs():
    """Outputs are fully overwritten: stale values in the buffers do not leak through."""
    inp = wl.random_lss_case(11, 1, 6, 16, 4, 8, 12, 30, 30, (-20.0, 20.0, -20.0, 20.0, -5.0, 3.0))
    say("[case] lss overwrite")
    dep, ctx, K, R, t = device_inputs(inp)
    out = torch.full((1, 16, 30, 30), 7.0, device="cuda")
    gd = torch.full_like(dep, 5.0)
    gc = torch.full_like(ctx, -3.0)
    ops.lss_forward(dep, ctx, K, R, t, inp.rng6, inp.X, inp.Y, inp.d_min, inp.d_step, out=out)
    ops.lss_backward(torch.from_numpy(inp.grad_out).cuda(), dep, ctx, K, R, t, inp.rng6, inp.X, inp.Y, inp.d_min,
                     inp.d_step, grad_depth=gd, grad_context=gc)
    torch.cuda.synchronize()
    ref = ls.lss_forward(inp.depth, inp.context, inp.K, inp.R, inp.t, inp.rng6, inp.X, inp.Y, inp.d_min,
                         inp.d_step)["out"]
    rd, rc = ls.lss_backward(inp.grad_out, inp.depth, inp.context, inp.K, inp.R, inp.t, inp.rng6, inp.X, inp.Y,
                             inp.d_min, inp.d_step)
    assert np.abs(out.cpu().numpy() - ref).max() <= 1e-4
    assert np.abs(gd.cpu().numpy().transpose(0, 1, 4, 2, 3) - rd).max() <= 1e-4
    assert np.abs(gc.cpu().numpy().transpose(0, 1, 4, 2, 3) - rc).max() <= 1e-4


def test_lss_degenerate_sizes():
    say("[case] lss degenerate sizes")
    base = wl.random_lss_case(13, 1, 6, 8, 4, 8, 6, 16, 16, (-20.0, 20.0, -20.0, 20.0, -5.0, 3.0))
    dep, ctx, K, R, t = device_inputs(base)
    g = torch.from_numpy(base.grad_out).cuda()
    a = (base.rng6, 16, 16, base.d_min, base.d_step)
    # no depth bins: no points, zero output and zero dL/dcontext
    dep0 = torch.empty((1, 6, 4, 8, 0), device="cuda")
    out = ops.lss_forward(dep0, ctx, K, R, t, *a)
    gd, gc = ops.lss_backward(g, dep0, ctx, K, R, t, *a, grad_context=torch.full_like(ctx, 9.0))
    torch.cuda.synchronize()
    assert not out.any() and gd.numel() == 0 and not gc.any()
    # no channels: empty output, zero dL/ddepth
    ctx0 = torch.empty((1, 6, 4, 8, 0), device="cuda")
    out = ops.lss_forward(dep, ctx0, K, R, t, *a)
    gd, gc = ops.lss_backward(torch.empty((1, 0, 16, 16), device="cuda"), dep, ctx0, K, R, t, *a,
                              grad_depth=torch.full_like(dep, 9.0))
    torch.cuda.synchronize()
    assert out.numel() == 0 and not gd.any() and gc.numel() == 0
    # no cameras: all-zero output
    e = torch.empty((1, 0, 4, 8, 6), device="cuda")
    ec = torch.empty((1, 0, 4, 8, 8), device="cuda")
    e3 = torch.empty((1, 0, 3, 3), device="cuda")
    out = ops.lss_forward(e, ec, e3, e3, torch.empty((1, 0, 3), device="cuda"), *a)
    torch.cuda.synchronize()
    assert out.shape == (1, 8, 16, 16) and not out.any()
    # empty batch
    out = ops.lss_forward(dep[:0], ctx[:0], K[:0], R[:0], t[:0], *a)
    torch.cuda.synchronize()
    assert out.shape == (0, 8, 16, 16)
