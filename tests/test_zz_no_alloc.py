"""GPU: fbev_backward_cameras_noalloc (the library's fixed device scratch instead of a caller
workspace) through the C ABI against fbev_backward_cameras (caller workspace) on the same inputs:
both run the same deterministic kernels, so the results must be bitwise equal.  Two calls in a
row, the second on a smaller problem (the scratch keeps the first call's partial sums, which the
second must not see), then the first problem again."""
import numpy as np
import pytest
import torch

from camera_bev_view_amd import _lib, ops
from camera_bev_view_amd import workloads as wl
from gpu_helpers import say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def both(inp):
    B, N, C, H, W = inp.F.shape
    F, K, R, t = to_device(inp)
    g = torch.from_numpy(inp.grad_out).cuda()
    ref = ops.camera_backward(g, F, K, R, t, inp.rng6, inp.X, inp.Y, inp.Z)
    out = tuple(torch.full_like(x, float("nan")) for x in ref)
    ops.camera_backward_noalloc(g, F, K, R, t, inp.rng6, inp.X, inp.Y, inp.Z, *out)
    torch.cuda.synchronize()
    return ref, out


@pytest.mark.parametrize("order", ["large then small", "small then large"])
def test_noalloc_matches_the_workspace_entry_point(order):
    big = wl.make_inputs("nuscenes", with_grad=True)
    small = wl.random_case(31, 1, 3, 16, 8, 22, 17, 23, 4, rng6=(-20.0, 20.0, -20.0, 20.0, -5.0, 3.0))
    seq = [big, small, big] if order == "large then small" else [small, big, small]
    for k, inp in enumerate(seq):
        say(f"[case] noalloc {order} call {k}: B,N,C,H,W={inp.F.shape} grid {inp.X}x{inp.Y}x{inp.Z}")
        ref, out = both(inp)
        for name, a, b in zip(("K", "R", "t"), ref, out):
            assert torch.equal(a, b), f"call {k}: dL/d{name} differs from fbev_backward_cameras"
        assert all(float(x.abs().max()) > 0 for x in ref)


def test_noalloc_allocates_nothing_and_rejects_oversize():
    inp = wl.make_inputs("nuscenes", with_grad=True)
    say("[case] noalloc: no torch allocation during the call; an oversize problem is refused")
    F, K, R, t = to_device(inp)
    g = torch.from_numpy(inp.grad_out).cuda()
    gK, gR, gt = (torch.empty(s, device="cuda") for s in ((1, 6, 3, 3), (1, 6, 3, 3), (1, 6, 3)))
    ops.camera_backward_noalloc(g, F, K, R, t, inp.rng6, inp.X, inp.Y, inp.Z, gK, gR, gt)   # first use on this device
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    alloc0 = torch.cuda.memory_allocated()
    free0 = torch.cuda.mem_get_info()[0]
    ops.camera_backward_noalloc(g, F, K, R, t, inp.rng6, inp.X, inp.Y, inp.Z, gK, gR, gt)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() == alloc0
    assert torch.cuda.mem_get_info()[0] == free0
    # 40 cameras of one sample need 40 * 12 * 8 * 1400 bytes (12 fp64 partial sums per camera and workgroup,
    # one workgroup per 32-cell unit of the 200 x 200 grid) > 4 MiB: refused before any launch
    big = wl.random_case(32, 1, 40, 4, 8, 22, 200, 200, 2, with_grad=True)
    F2, K2, R2, t2 = to_device(big)
    g2 = torch.from_numpy(big.grad_out).cuda()
    o2 = (torch.empty((1, 40, 3, 3), device="cuda"), torch.empty((1, 40, 3, 3), device="cuda"),
          torch.empty((1, 40, 3), device="cuda"))
    with pytest.raises(_lib.FlashBevError, match="allocation-free variant holds"):
        ops.camera_backward_noalloc(g2, F2, K2, R2, t2, big.rng6, 200, 200, 2, *o2)
