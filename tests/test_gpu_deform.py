"""GPU: the Deformable Aggregation entry points (fbev_deform_forward /
fbev_deform_backward) against the fp64 oracle (oracle.deform_agg).

Parity rules:
  * forward within |d| <= 1e-4 + 1e-5 |ref|, except queries with a (camera,
    keypoint) sample within 1e-4 px of an image edge (a rounding flip of the
    in-view test changes the whole sample);
  * dL/dweights element-wise within 1e-4 + 1e-5 |ref| away from such samples;
  * dL/dfeatures, dL/doffsets and dL/danchors within 1e-3 relative L2 (and
    element-wise within 1e-4 + 1e-5 max|ref| away from near-edge keypoints for
    the offsets).
Every case prints its label before the GPU work starts.
"""
import numpy as np
import pytest
import torch

import oracle.deform_agg as da
from camera_bev_view_amd import ops
from camera_bev_view_amd import workloads as wl
from gpu_helpers import ATOL, BWD_REL_L2, RTOL, rel_l2, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def to_dev(inp):
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return (dev(inp.F.transpose(0, 1, 3, 4, 2)), dev(inp.K), dev(inp.R), dev(inp.t), dev(inp.anchors),
            dev(inp.offsets), dev(inp.weights))


def deform_parity(inp, label, backward=True):
    B, N, C, H, W = inp.F.shape
    Q, Kp = inp.offsets.shape[1:3]
    say(f"[case] deform {label}: B,N,C={B},{N},{C} HxW={H}x{W} Q={Q} Kp={Kp}")
    F, K, R, t, A, D, Wt = to_dev(inp)
    out = ops.deform_forward(F, K, R, t, A, D, Wt)
    torch.cuda.synchronize()
    ref = da.deform_forward(inp.F, inp.K, inp.R, inp.t, inp.anchors, inp.offsets, inp.weights)
    near = ref["near_edge"]                                        # [B, N, Q, K]
    q_ok = ~near.any(axis=(1, 3))                                   # [B, Q]
    got = out.cpu().numpy()
    diff = np.abs(got - ref["out"])
    bad = (diff > ATOL + RTOL * np.abs(ref["out"])) & q_ok[..., None]
    say(f"[parity] deform {label}: forward max|d|={diff[q_ok].max(initial=0):.3e} in-view samples="
        f"{int(ref['valid'].sum())} near-edge samples={int(near.sum())}")
    assert not bad.any(), f"{label}: {int(bad.sum())} outputs outside tolerance, worst {diff[bad].max():.3e}"
    if not backward:
        return
    gF, gW, gO, gA = ops.deform_backward(torch.from_numpy(inp.grad_out).cuda(), F, K, R, t, A, D, Wt)
    torch.cuda.synchronize()
    rF, rW, rO, rA = da.deform_backward(inp.grad_out, inp.F, inp.K, inp.R, inp.t, inp.anchors, inp.offsets,
                                        inp.weights)
    gF = gF.cpu().numpy().transpose(0, 1, 4, 2, 3)
    gW, gO, gA = gW.cpu().numpy(), gO.cpu().numpy(), gA.cpu().numpy()
    eF, eO, eA = rel_l2(gF, rF), rel_l2(gO, rO), rel_l2(gA, rA)
    say(f"[parity] deform {label}: backward rel L2 features {eF:.3e} offsets {eO:.3e} anchors {eA:.3e} "
        f"weights max|d| {np.abs(gW - rW).max(initial=0):.3e}")
    for name, e, r in (("features", eF, rF), ("offsets", eO, rO), ("anchors", eA, rA)):
        if np.linalg.norm(r) > 0:
            assert e <= BWD_REL_L2, f"{label}: dL/d{name} rel L2 {e:.3e}"
    w_ok = ~near.transpose(0, 2, 1, 3)                              # [B, Q, N, K]
    bad_w = (np.abs(gW - rW) > ATOL + RTOL * np.abs(rW)) & w_ok
    assert not bad_w.any(), f"{label}: {int(bad_w.sum())} dL/dweights outside tolerance"
    k_ok = ~near.any(axis=1)                                        # [B, Q, K]
    tol_o = ATOL + RTOL * max(1.0, np.abs(rO).max(initial=0))
    ratio_o = float((np.abs(gO - rO) * k_ok[..., None]).max(initial=0) / tol_o)
    say(f"[parity] deform {label}: dL/doffsets worst |d| / (1e-4 + 1e-5 max|ref|) = {ratio_o:.3f}")
    bad_o = (np.abs(gO - rO) > tol_o) & k_ok[..., None]
    assert not bad_o.any(), f"{label}: {int(bad_o.sum())} dL/doffsets outside tolerance"


def test_deform_sparse_queries():
    """900 queries x 13 keypoints, C = 256, six cameras, 16 x 44 maps."""
    deform_parity(wl.make_deform_inputs("deform", with_grad=True), "sparse queries")


def test_deform_dense_bev_queries():
    """One query per cell of a 200 x 200 grid, 8 keypoints up the pillar, C = 64."""
    deform_parity(wl.make_deform_inputs("deform_bev", with_grad=True), "dense BEV queries")


DEFORM_CASES = [
    # label, B, N, C, H, W, Q, Kp, spread, offset sigma, pitch
    ("ragged channels and queries", 2, 6, 70, 8, 22, 37, 5, 20.0, 1.5, 0.0),
    ("two channel blocks", 1, 6, 300, 6, 14, 21, 3, 25.0, 1.0, 5.0),
    ("many keypoints: four passes of 64 pairs", 1, 6, 32, 8, 22, 19, 40, 20.0, 2.0, -4.0),
    ("one camera, one keypoint, one channel", 2, 1, 1, 5, 9, 17, 1, 8.0, 0.5, 0.0),
    ("64 cameras", 1, 64, 16, 4, 8, 23, 2, 15.0, 1.0, 0.0),
    ("1x1 maps", 1, 6, 8, 1, 1, 16, 4, 10.0, 1.0, 0.0),
]


@pytest.mark.parametrize("case", DEFORM_CASES, ids=[c[0] for c in DEFORM_CASES])
def test_deform_cases(case):
    label, B, N, C, H, W, Q, Kp, spread, sigma, pitch = case
    inp = wl.random_deform_case(len(label), B, N, C, H, W, Q, Kp, spread, sigma, pitch)
    deform_parity(inp, label)


def test_deform_constant_features_and_determinism():
    inp = wl.random_deform_case(3, 1, 6, 24, 8, 22, 50, 6)
    say("[case] deform constant features")
    inp.F[:] = 2.5
    F, K, R, t, A, D, Wt = to_dev(inp)
    a = ops.deform_forward(F, K, R, t, A, D, Wt)
    b = ops.deform_forward(F, K, R, t, A, D, Wt)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    ref = da.deform_forward(inp.F, inp.K, inp.R, inp.t, inp.anchors, inp.offsets, inp.weights)
    expect = 2.5 * (inp.weights * ref["valid"].transpose(0, 2, 1, 3)).sum(axis=(2, 3))
    ok = ~ref["near_edge"].any(axis=(1, 3))
    assert np.abs(a.cpu().numpy()[..., 0] - expect)[ok].max(initial=0) <= 1e-5


def test_deform_degenerate_sizes():
    say("[case] deform degenerate sizes")
    inp = wl.random_deform_case(5, 1, 6, 8, 8, 22, 10, 3)
    F, K, R, t, A, D, Wt = to_dev(inp)
    g = torch.from_numpy(inp.grad_out).cuda()
    # no keypoints: zero output, zero anchor gradient
    D0 = torch.empty((1, 10, 0, 3), device="cuda")
    W0 = torch.empty((1, 10, 6, 0), device="cuda")
    out = ops.deform_forward(F, K, R, t, A, D0, W0)
    gF, gW, gO, gA = ops.deform_backward(g, F, K, R, t, A, D0, W0)
    torch.cuda.synchronize()
    assert not out.any() and not gF.any() and gW.numel() == 0 and gO.numel() == 0 and not gA.any()
    # no queries
    out = ops.deform_forward(F, K, R, t, A[:, :0], D[:, :0], Wt[:, :0])
    torch.cuda.synchronize()
    assert out.shape == (1, 0, 8)
    # no channels: empty output, zero gradients
    Fc = torch.empty((1, 6, 8, 22, 0), device="cuda")
    gF, gW, gO, gA = ops.deform_backward(torch.empty((1, 10, 0), device="cuda"), Fc, K, R, t, A, D, Wt)
    torch.cuda.synchronize()
    assert gF.numel() == 0 and not gW.any() and not gO.any() and not gA.any()


def test_deform_many_pixels_two_kernel_scan():
    """More than 16 scan blocks of 16 384 pixels (2 x 6 x 128 x 176 = 270 336): the bucket offsets come from
    the two-launch scan (block sums, then the blocks' own scans)."""
    deform_parity(wl.random_deform_case(21, 2, 6, 4, 128, 176, 40, 4, spread=20.0), "270k pixels, two-launch scan")


def test_deform_unaligned_upstream_uses_lane_per_channel_gather():
    """An upstream gradient that is not 16-byte aligned takes the lanes = channels paths (the per-sample sums
    and the dL/dF gather); its gradients match the 16-byte paths' (dL/dw and dL/doffsets up to the order of
    the channel sums, dL/dF up to the bucket order) and the oracle."""
    inp = wl.random_deform_case(22, 1, 6, 16, 16, 44, 120, 6)
    say("[case] deform unaligned upstream gradient")
    F, K, R, t, A, D, Wt = to_dev(inp)
    g = torch.from_numpy(inp.grad_out).cuda()
    big = torch.empty(g.numel() + 1, dtype=torch.float32, device="cuda")
    g_off = big[1:].view(g.shape)
    g_off.copy_(g)
    assert g_off.is_contiguous() and g_off.data_ptr() % 16 != 0
    gF4, gW4, gO4, _ = ops.deform_backward(g, F, K, R, t, A, D, Wt)
    gF1, gW1, gO1, _ = ops.deform_backward(g_off, F, K, R, t, A, D, Wt)
    torch.cuda.synchronize()
    for a4, a1 in ((gW4, gW1), (gO4, gO1)):
        bound = 1e-6 + 1e-5 * a4.abs().max().item()
        assert (a4 - a1).abs().max().item() <= bound
    assert torch.allclose(gF4, gF1, rtol=1e-5, atol=1e-6)
    rF, _, _, _ = da.deform_backward(inp.grad_out, inp.F, inp.K, inp.R, inp.t, inp.anchors, inp.offsets, inp.weights)
    assert rel_l2(gF1.cpu().numpy().transpose(0, 1, 4, 2, 3), rF) <= BWD_REL_L2
