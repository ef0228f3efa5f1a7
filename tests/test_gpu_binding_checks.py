"""GPU: the binding refuses caller buffers that live off the inputs' device (or have
the wrong dtype) with a ValueError before anything is launched."""
import numpy as np
import pytest
import torch

from camera_bev_view_amd import ops
from camera_bev_view_amd import workloads as wl
from gpu_helpers import say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def test_host_out_and_grad_buffers_are_refused():
    inp = wl.random_case(3, 1, 6, 8, 8, 22, 6, 7, 3, rng6=(-20.0, 20.0, -20.0, 20.0, -5.0, 3.0))
    say("[case] binding checks: out / grad_out / workspace on the wrong device or dtype")
    F, K, R, t = to_device(inp)
    B, N, H, W, C = F.shape
    g_host = torch.from_numpy(inp.grad_out)
    with pytest.raises(ValueError, match="out must be"):
        ops.forward(F, K, R, t, inp.rng6, 6, 7, 3, out=torch.empty((B, C, 6, 7)))
    with pytest.raises(ValueError, match="grad_out must be a device tensor"):
        ops.backward(g_host, (B, N, H, W, C), K, R, t, inp.rng6, 6, 7, 3)
    with pytest.raises(ValueError, match="grad_out must be a device tensor"):
        ops.camera_backward(g_host, F, K, R, t, inp.rng6, 6, 7, 3)
    g = g_host.cuda()
    with pytest.raises(ValueError, match="workspace must be"):
        ops.camera_backward(g, F, K, R, t, inp.rng6, 6, 7, 3, workspace=torch.empty(1 << 16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="workspace must be"):
        ops.camera_backward(g, F, K, R, t, inp.rng6, 6, 7, 3,
                            workspace=torch.empty(1 << 16, dtype=torch.float32, device="cuda"))
    prev = torch.zeros((B, 2, 6, 7), device="cuda")
    ego = torch.tensor([[[1.0, 0.0, 0.0], [0.0, 1.0, 0.0]]], device="cuda")
    with pytest.raises(ValueError, match="out must be"):
        ops.forward_temporal(F, K, R, t, inp.rng6, 6, 7, 3, prev, ego, out=torch.empty((B, C + 2, 6, 7)))
    with pytest.raises(ValueError, match="grad_out must be a device tensor"):
        ops.backward_temporal(torch.zeros((B, C + 2, 6, 7)), (B, N, H, W, C), K, R, t, inp.rng6, 6, 7, 3, 2, ego)
    packed = ops.pack_levels([F])
    with pytest.raises(ValueError, match="out must be"):
        ops.forward_levels(packed, [(H, W)], K, R, t, inp.rng6, 6, 7, 3, out=torch.empty((B, C, 6, 7)))
    with pytest.raises(ValueError, match="grad_out must be a device tensor"):
        ops.backward_levels(g_host, B, N, C, [(H, W)], K, R, t, inp.rng6, 6, 7, 3)


def test_deform_and_lss_buffers_are_refused():
    di = wl.random_deform_case(4, 1, 6, 16, 8, 22, 5, 3)
    say("[case] binding checks: deformable and Lift-Splat buffers")
    dvc = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    args = (dvc(di.F.transpose(0, 1, 3, 4, 2)), dvc(di.K), dvc(di.R), dvc(di.t), dvc(di.anchors), dvc(di.offsets),
            dvc(di.weights))
    with pytest.raises(ValueError, match="out must be"):
        ops.deform_forward(*args, out=torch.empty((1, 5, 16)))
    with pytest.raises(ValueError, match="workspace must be"):
        ops.deform_backward(dvc(di.grad_out), *args, workspace=torch.empty(1 << 16, dtype=torch.uint8))
    si = wl.random_lss_case(2, 1, 6, 8, 4, 11, 9, 12, 10, (-20.0, 20.0, -20.0, 20.0, -5.0, 3.0))
    dep = dvc(si.depth.transpose(0, 1, 3, 4, 2))
    ctx = dvc(si.context.transpose(0, 1, 3, 4, 2))
    with pytest.raises(ValueError, match="out must be"):
        ops.lss_forward(dep, ctx, dvc(si.K), dvc(si.R), dvc(si.t), si.rng6, si.X, si.Y, si.d_min, si.d_step,
                        out=torch.empty((1, 8, si.X, si.Y)))
