"""GPU: the multi-level (feature-pyramid) entry points against the multi-level oracle.

Every case prints its label before the GPU work starts.  Parity rules are
those of gpu_helpers (counts bit-exact away from level-0 image edges, outputs
within 1e-4 + 1e-5 |ref|, gradients within 1e-3 relative L2).
"""
import numpy as np
import pytest
import torch

import oracle.multilevel as ml
from camera_bev_view_amd import ops
from camera_bev_view_amd import workloads as wl
from gpu_helpers import BWD_REL_L2, check_forward, rel_l2, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def device_inputs(inp):
    """Packed channels-last level features [B,N,P,C] plus fp32 K, R, t on the GPU."""
    lv = [torch.from_numpy(np.ascontiguousarray(F.transpose(0, 1, 3, 4, 2))) for F in inp.levels]
    if inp.dtype == "bf16":
        lv = [x.to(torch.bfloat16) for x in lv]
    packed = ops.pack_levels([x.cuda() for x in lv])
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return packed, dev(inp.K), dev(inp.R), dev(inp.t)


def levels_forward_parity(inp, label, rows=None):
    B, N, C = inp.levels[0].shape[:3]
    say(f"[case] levels {label}: B,N,C={B},{N},{C} levels={list(inp.shapes)} X,Y,Z={inp.X},{inp.Y},{inp.Z} "
        f"dtype={inp.dtype}")
    packed, K, R, t = device_inputs(inp)
    out, cnt = ops.forward_levels(packed, inp.shapes, K, R, t, inp.rng6, inp.X, inp.Y, inp.Z, with_counts=True)
    torch.cuda.synchronize()
    ref = ml.oracle_forward_levels(inp.levels, inp.K, inp.R, inp.t, inp.rng6, inp.X, inp.Y, inp.Z, rows=rows)
    check_forward(out, cnt, ref, rows=rows, label=label)
    return out, cnt, ref


def levels_backward_parity(inp, label):
    B, N, C = inp.levels[0].shape[:3]
    say(f"[case] levels backward {label}: levels={list(inp.shapes)} X,Y,Z={inp.X},{inp.Y},{inp.Z}")
    _, K, R, t = device_inputs(inp)
    g = ops.backward_levels(torch.from_numpy(inp.grad_out).cuda(), B, N, C, inp.shapes, K, R, t, inp.rng6,
                            inp.X, inp.Y, inp.Z)
    torch.cuda.synchronize()
    got = [x.cpu().numpy().transpose(0, 1, 4, 2, 3) for x in ops.unpack_levels(g, inp.shapes)]
    ref = ml.oracle_backward_levels(inp.grad_out, inp.K, inp.R, inp.t, inp.rng6, inp.X, inp.Y, inp.Z, inp.shapes)
    err = rel_l2(np.concatenate([a.ravel() for a in got]), np.concatenate([r.ravel() for r in ref]))
    say(f"[parity] levels backward {label}: rel L2 = {err:.3e}")
    assert err <= BWD_REL_L2
    for a, r in zip(got, ref):
        assert np.abs(a - r).max() <= 1e-4 + 1e-5 * np.abs(r).max()


def test_pyramid_workload():
    inp = wl.make_level_inputs("pyramid", with_grad=True)
    levels_forward_parity(inp, "pyramid 1x6x64 32x88/16x44/8x22 -> 200x200x8")
    levels_backward_parity(inp, "pyramid")


LEVEL_CASES = [
    # dtype, B, N, C, H, W, ratios, X, Y, Z
    ("f32", 1, 6, 16, 16, 44, (1, 2), 17, 37, 5),
    ("bf16", 2, 6, 24, 32, 88, (1, 2, 4, 8), 9, 45, 6),
    ("f32", 1, 16, 8, 8, 24, (1, 2, 4, 8), 7, 19, 4),      # N * L = 64, one bin per item
    ("f32", 1, 6, 20, 16, 44, (1, 4, 2), 11, 33, 24),       # ratios in any order; forward merges rows
    ("f32", 2, 3, 64, 16, 48, (1, 1, 2), 13, 21, 9),        # a repeated level
]


@pytest.mark.parametrize("case", LEVEL_CASES, ids=lambda c: "x".join(str(v) for v in c[:6]) + "-r" +
                         "".join(map(str, c[6])) + "-" + "x".join(map(str, c[7:])))
def test_ragged_levels(case):
    dt, B, N, C, H, W, ratios, X, Y, Z = case
    inp = wl.random_level_case(sum(ratios) + X + Y, B, N, C, H, W, ratios, X, Y, Z,
                               rng6=(-25.0, 25.0, -25.0, 25.0, -5.0, 3.0), dtype=dt)
    levels_forward_parity(inp, str(case))
    if dt == "f32":
        levels_backward_parity(inp, str(case))


def test_one_level_matches_single_level_entry_point():
    inp = wl.make_inputs("nuscenes")
    say("[case] levels: L = 1 through fbev_forward_levels equals fbev_forward")
    F = torch.from_numpy(np.ascontiguousarray(inp.F.transpose(0, 1, 3, 4, 2))).cuda()
    K, R, t = (torch.from_numpy(a).cuda() for a in (inp.K, inp.R, inp.t))
    a, ca = ops.forward(F, K, R, t, inp.rng6, inp.X, inp.Y, inp.Z, with_counts=True)
    B, N, H, W, C = F.shape
    b, cb = ops.forward_levels(F.reshape(B, N, H * W, C), [(H, W)], K, R, t, inp.rng6, inp.X, inp.Y, inp.Z,
                               with_counts=True)
    torch.cuda.synchronize()
    assert torch.equal(ca, cb) and torch.equal(a, b)


def test_constant_levels_on_gpu():
    inp = wl.random_level_case(3, 1, 6, 8, 16, 44, (1, 2, 4), 25, 31, 6, rng6=(-25.0, 25.0, -25.0, 25.0, -5.0, 3.0))
    consts = (1.5, -0.25, 2.0)
    inp.levels = [np.full_like(F, c) for F, c in zip(inp.levels, consts)]
    say("[case] levels: constant maps per level give the mean constant per bin seen")
    packed, K, R, t = device_inputs(inp)
    out, cnt = ops.forward_levels(packed, inp.shapes, K, R, t, inp.rng6, inp.X, inp.Y, inp.Z, with_counts=True)
    torch.cuda.synchronize()
    nz = (cnt >= 1).sum(-1).float()
    assert torch.allclose(out, float(np.mean(consts)) * nz[:, None].expand_as(out), rtol=1e-6, atol=1e-5)
