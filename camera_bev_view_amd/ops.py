"""PyTorch-facing calls of libflashbev: argument marshalling only.

PyTorch supplies device memory and the current HIP stream; every step of the
view transform runs in the library's kernels.  Names follow the notation of
the FlashBEV reading notes: features F with B samples, N cameras, C channels
on an H x W map; a BEV grid of X x Y cells and Z height bins.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple

import torch

from . import _lib

_DTYPES = {torch.float32: _lib.FBEV_DTYPE_F32, torch.bfloat16: _lib.FBEV_DTYPE_BF16}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None or t.numel() == 0 else t.data_ptr()


def _check_cams(K: torch.Tensor, R: torch.Tensor, t: torch.Tensor, B: int, N: int, device) -> None:
    for name, x, shape in (("K", K, (B, N, 3, 3)), ("R", R, (B, N, 3, 3)), ("t", t, (B, N, 3))):
        if tuple(x.shape) != shape:
            raise ValueError(f"{name} must have shape {shape}, got {tuple(x.shape)}")
        if x.dtype != torch.float32 or not x.is_contiguous() or x.device != device:
            raise ValueError(f"{name} must be a contiguous float32 tensor on {device}")


def _check_device_tensor(name: str, x: torch.Tensor, device=None) -> None:
    """x must live in device memory (on ``device`` when given): the library dereferences it on the GPU."""
    if not x.is_cuda or (device is not None and x.device != device):
        raise ValueError(f"{name} must be a device tensor" + (f" on {device}" if device is not None else ""))


def _check_out(name: str, out: torch.Tensor, shape, device) -> None:
    if tuple(out.shape) != tuple(shape) or out.dtype != torch.float32 or not out.is_contiguous() \
            or out.device != device:
        raise ValueError(f"{name} must be a contiguous float32 {list(shape)} tensor on {device}")


def _check_workspace(ws: torch.Tensor, device) -> None:
    if ws.dtype != torch.uint8 or not ws.is_contiguous() or ws.device != device:
        raise ValueError(f"workspace must be a contiguous uint8 tensor on {device}")


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def forward(features: torch.Tensor, K: torch.Tensor, R: torch.Tensor, t: torch.Tensor,
            bev_range: Sequence[float], X: int, Y: int, Z: int, *, with_counts: bool = False,
            out: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """fbev_forward on channels-last features [B,N,H,W,C] (fp32 or bf16).

    Returns (out [B,C,X,Y] fp32, counts [B,X,Y,Z] uint8 or None).
    """
    if features.dim() != 5:
        raise ValueError("features must be [B,N,H,W,C]")
    if features.dtype not in _DTYPES:
        raise ValueError(f"unsupported feature dtype {features.dtype}")
    if not features.is_cuda or not features.is_contiguous():
        raise ValueError("features must be a contiguous device tensor")
    B, N, H, W, C = features.shape
    dev = features.device
    _check_cams(K, R, t, B, N, dev)
    if out is None:
        out = torch.empty((B, C, X, Y), dtype=torch.float32, device=dev)
    else:
        _check_out("out", out, (B, C, X, Y), dev)
    counts = torch.empty((B, X, Y, Z), dtype=torch.uint8, device=dev) if with_counts else None
    lib = _lib.load()
    _lib.check(lib.fbev_forward(_ptr(features), _DTYPES[features.dtype], _lib.feat_desc(B, N, C, H, W),
                                _ptr(K), _ptr(R), _ptr(t), _lib.bev_range(bev_range), X, Y, Z,
                                _ptr(out), _ptr(counts), _stream(dev)))
    return out, counts


def backward(grad_out: torch.Tensor, feat_shape: Sequence[int], K: torch.Tensor, R: torch.Tensor,
             t: torch.Tensor, bev_range: Sequence[float], X: int, Y: int, Z: int) -> torch.Tensor:
    """fbev_backward: dL/dF as fp32 channels-last [B,N,H,W,C] from grad_out [B,C,X,Y]."""
    B, N, H, W, C = (int(v) for v in feat_shape)
    if tuple(grad_out.shape) != (B, C, X, Y) or grad_out.dtype != torch.float32:
        raise ValueError("grad_out must be float32 [B,C,X,Y]")
    _check_device_tensor("grad_out", grad_out)
    grad_out = grad_out.contiguous()
    dev = grad_out.device
    _check_cams(K, R, t, B, N, dev)
    gF = torch.empty((B, N, H, W, C), dtype=torch.float32, device=dev)
    lib = _lib.load()
    _lib.check(lib.fbev_backward(_ptr(grad_out), _lib.feat_desc(B, N, C, H, W), _ptr(K), _ptr(R), _ptr(t),
                                 _lib.bev_range(bev_range), X, Y, Z, _ptr(gF), _stream(dev)))
    return gF


def camera_backward(grad_out: torch.Tensor, features: torch.Tensor, K: torch.Tensor, R: torch.Tensor,
                    t: torch.Tensor, bev_range: Sequence[float], X: int, Y: int, Z: int,
                    workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """fbev_backward_cameras: (dL/dK [B,N,3,3], dL/dR [B,N,3,3], dL/dt [B,N,3]) of L = <grad_out, out>
    for fp32 channels-last features [B,N,H,W,C].  ``workspace`` (a uint8 device tensor) is allocated when
    not given or too small."""
    if features.dim() != 5 or features.dtype != torch.float32 or not features.is_cuda or not features.is_contiguous():
        raise ValueError("features must be a contiguous float32 device tensor [B,N,H,W,C]")
    B, N, H, W, C = features.shape
    dev = features.device
    if tuple(grad_out.shape) != (B, C, X, Y) or grad_out.dtype != torch.float32:
        raise ValueError("grad_out must be float32 [B,C,X,Y]")
    _check_device_tensor("grad_out", grad_out, dev)
    grad_out = grad_out.contiguous()
    _check_cams(K, R, t, B, N, dev)
    lib = _lib.load()
    fd = _lib.feat_desc(B, N, C, H, W)
    need = ctypes.c_size_t(0)
    _lib.check(lib.fbev_backward_cameras_workspace(fd, X, Y, Z, ctypes.byref(need)))
    if workspace is not None:
        _check_workspace(workspace, dev)
    if workspace is None or workspace.numel() < need.value:
        workspace = torch.empty((max(need.value, 1),), dtype=torch.uint8, device=dev)
    gK = torch.empty((B, N, 3, 3), dtype=torch.float32, device=dev)
    gR = torch.empty((B, N, 3, 3), dtype=torch.float32, device=dev)
    gt = torch.empty((B, N, 3), dtype=torch.float32, device=dev)
    _lib.check(lib.fbev_backward_cameras(_ptr(grad_out), _ptr(features), fd, _ptr(K), _ptr(R), _ptr(t),
                                         _lib.bev_range(bev_range), X, Y, Z, _ptr(gK), _ptr(gR), _ptr(gt),
                                         _ptr(workspace), workspace.numel(), _stream(dev)))
    return gK, gR, gt


def camera_backward_noalloc(grad_out: torch.Tensor, features: torch.Tensor, K: torch.Tensor, R: torch.Tensor,
                            t: torch.Tensor, bev_range: Sequence[float], X: int, Y: int, Z: int,
                            grad_K: torch.Tensor, grad_R: torch.Tensor, grad_t: torch.Tensor) -> None:
    """fbev_backward_cameras_noalloc: camera_backward into the caller's grad_K [B,N,3,3], grad_R [B,N,3,3] and
    grad_t [B,N,3] with the library's fixed device scratch instead of a workspace (nothing is allocated)."""
    if features.dim() != 5 or features.dtype != torch.float32 or not features.is_cuda or not features.is_contiguous():
        raise ValueError("features must be a contiguous float32 device tensor [B,N,H,W,C]")
    B, N, H, W, C = features.shape
    dev = features.device
    if tuple(grad_out.shape) != (B, C, X, Y) or grad_out.dtype != torch.float32 or not grad_out.is_contiguous():
        raise ValueError("grad_out must be a contiguous float32 [B,C,X,Y] tensor")
    _check_device_tensor("grad_out", grad_out, dev)
    _check_cams(K, R, t, B, N, dev)
    for name, x, shape in (("grad_K", grad_K, (B, N, 3, 3)), ("grad_R", grad_R, (B, N, 3, 3)),
                           ("grad_t", grad_t, (B, N, 3))):
        _check_out(name, x, shape, dev)
    lib = _lib.load()
    _lib.check(lib.fbev_backward_cameras_noalloc(_ptr(grad_out), _ptr(features), _lib.feat_desc(B, N, C, H, W),
                                                 _ptr(K), _ptr(R), _ptr(t), _lib.bev_range(bev_range), X, Y, Z,
                                                 _ptr(grad_K), _ptr(grad_R), _ptr(grad_t), _stream(dev)))


class SamplingVT(torch.autograd.Function):
    """Autograd wrapper: gradients with respect to the features and, for fp32 features, the cameras."""

    @staticmethod
    def forward(ctx, features, K, R, t, bev_range, X, Y, Z):
        out, _ = forward(features, K, R, t, bev_range, X, Y, Z)
        ctx.save_for_backward(features, K, R, t)
        ctx.meta = (tuple(features.shape), features.dtype, tuple(bev_range), X, Y, Z)
        return out

    @staticmethod
    def backward(ctx, grad_out):
        features, K, R, t = ctx.saved_tensors
        shape, dtype, rng, X, Y, Z = ctx.meta
        g = grad_out.float().contiguous()
        gF = backward(g, shape, K, R, t, rng, X, Y, Z).to(dtype) if ctx.needs_input_grad[0] else None
        gK = gR = gt = None
        if any(ctx.needs_input_grad[1:4]):
            if dtype != torch.float32:
                raise NotImplementedError("camera gradients need float32 features")
            gK, gR, gt = camera_backward(g, features, K, R, t, rng, X, Y, Z)
        return gF, gK, gR, gt, None, None, None, None


def bev_sample(features: torch.Tensor, K: torch.Tensor, R: torch.Tensor, t: torch.Tensor,
               bev_range: Sequence[float], X: int, Y: int, Z: int, channels_last: bool = True) -> torch.Tensor:
    """Differentiable Sampling-VT.  ``channels_last=False`` accepts [B,N,C,H,W] and
    permutes it to the library's [B,N,H,W,C] layout first (one copy)."""
    if not channels_last:
        features = features.permute(0, 1, 3, 4, 2).contiguous()
    return SamplingVT.apply(features, K, R, t, tuple(bev_range), X, Y, Z)


# ---- temporal fusion (fbev_forward_temporal / fbev_backward_temporal)

def _check_temporal(prev_bev: torch.Tensor, ego: torch.Tensor, B: int, X: int, Y: int, device) -> int:
    if prev_bev.dim() != 4 or prev_bev.shape[0] != B or tuple(prev_bev.shape[2:]) != (X, Y):
        raise ValueError(f"prev_bev must be [B={B}, Cp, X={X}, Y={Y}], got {tuple(prev_bev.shape)}")
    if prev_bev.dtype != torch.float32 or not prev_bev.is_contiguous() or prev_bev.device != device:
        raise ValueError(f"prev_bev must be a contiguous float32 tensor on {device}")
    if tuple(ego.shape) != (B, 2, 3) or ego.dtype != torch.float32 or not ego.is_contiguous() or ego.device != device:
        raise ValueError(f"ego must be a contiguous float32 [B, 2, 3] tensor on {device}")
    return int(prev_bev.shape[1])


def forward_temporal(features: torch.Tensor, K: torch.Tensor, R: torch.Tensor, t: torch.Tensor,
                     bev_range: Sequence[float], X: int, Y: int, Z: int, prev_bev: torch.Tensor, ego: torch.Tensor,
                     *, with_counts: bool = False, out: Optional[torch.Tensor] = None
                     ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """fbev_forward_temporal: out [B, C + Cp, X, Y] = the current frame's Sampling-VT channels, then the previous
    BEV map prev_bev [B, Cp, X, Y] resampled at the current cells moved by ego [B, 2, 3] (current -> previous
    ego x, y).  Returns (out, counts or None)."""
    if features.dim() != 5 or features.dtype not in _DTYPES or not features.is_cuda or not features.is_contiguous():
        raise ValueError("features must be a contiguous fp32 or bf16 device tensor [B,N,H,W,C]")
    B, N, H, W, C = features.shape
    dev = features.device
    _check_cams(K, R, t, B, N, dev)
    Cp = _check_temporal(prev_bev, ego, B, X, Y, dev)
    if out is None:
        out = torch.empty((B, C + Cp, X, Y), dtype=torch.float32, device=dev)
    else:
        _check_out("out", out, (B, C + Cp, X, Y), dev)
    counts = torch.empty((B, X, Y, Z), dtype=torch.uint8, device=dev) if with_counts else None
    lib = _lib.load()
    _lib.check(lib.fbev_forward_temporal(_ptr(features), _DTYPES[features.dtype], _lib.feat_desc(B, N, C, H, W),
                                         _ptr(K), _ptr(R), _ptr(t), _lib.bev_range(bev_range), X, Y, Z,
                                         _ptr(prev_bev), Cp, _ptr(ego), _ptr(out), _ptr(counts), _stream(dev)))
    return out, counts


def backward_temporal(grad_out: torch.Tensor, feat_shape: Sequence[int], K: torch.Tensor, R: torch.Tensor,
                      t: torch.Tensor, bev_range: Sequence[float], X: int, Y: int, Z: int, Cp: int,
                      ego: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """fbev_backward_temporal: (dL/dF [B,N,H,W,C] fp32, dL/dprev_bev [B,Cp,X,Y]) from grad_out [B, C + Cp, X, Y]."""
    B, N, H, W, C = (int(v) for v in feat_shape)
    if tuple(grad_out.shape) != (B, C + Cp, X, Y) or grad_out.dtype != torch.float32:
        raise ValueError("grad_out must be float32 [B, C + Cp, X, Y]")
    _check_device_tensor("grad_out", grad_out)
    grad_out = grad_out.contiguous()
    dev = grad_out.device
    _check_cams(K, R, t, B, N, dev)
    if tuple(ego.shape) != (B, 2, 3) or ego.dtype != torch.float32 or not ego.is_contiguous() or ego.device != dev:
        raise ValueError(f"ego must be a contiguous float32 [B, 2, 3] tensor on {dev}")
    gF = torch.empty((B, N, H, W, C), dtype=torch.float32, device=dev)
    gP = torch.empty((B, Cp, X, Y), dtype=torch.float32, device=dev)
    lib = _lib.load()
    _lib.check(lib.fbev_backward_temporal(_ptr(grad_out), _lib.feat_desc(B, N, C, H, W), _ptr(K), _ptr(R), _ptr(t),
                                          _lib.bev_range(bev_range), X, Y, Z, Cp, _ptr(ego), _ptr(gF), _ptr(gP),
                                          _stream(dev)))
    return gF, gP


class TemporalVT(torch.autograd.Function):
    """Autograd wrapper of the temporal fused transform: gradients for the features and the previous map."""

    @staticmethod
    def forward(ctx, features, prev_bev, K, R, t, ego, bev_range, X, Y, Z):
        out, _ = forward_temporal(features, K, R, t, bev_range, X, Y, Z, prev_bev, ego)
        ctx.save_for_backward(K, R, t, ego)
        ctx.meta = (tuple(features.shape), features.dtype, int(prev_bev.shape[1]), tuple(bev_range), X, Y, Z)
        return out

    @staticmethod
    def backward(ctx, grad_out):
        K, R, t, ego = ctx.saved_tensors
        shape, dtype, Cp, rng, X, Y, Z = ctx.meta
        gF, gP = backward_temporal(grad_out.float(), shape, K, R, t, rng, X, Y, Z, Cp, ego)
        return gF.to(dtype), gP, None, None, None, None, None, None, None, None


# ---- feature pyramids (fbev_forward_levels / fbev_backward_levels)

def level_ratios(H: int, W: int, shapes: Sequence[Sequence[int]]) -> Tuple[int, ...]:
    """Integer ratios r_l of level shapes [(H_l, W_l), ...] to the level-0 map H x W."""
    ratios = []
    for (h, w) in shapes:
        if h <= 0 or w <= 0 or H % h or W % w or H // h != W // w:
            raise ValueError(f"level {h}x{w} is not an integer downscale of {H}x{W}")
        ratios.append(H // h)
    return tuple(ratios)


def pack_levels(levels: Sequence[torch.Tensor]) -> torch.Tensor:
    """[B,N,H_l,W_l,C] level maps -> the packed [B,N,P,C] layout (one copy)."""
    B, N, _, _, C = levels[0].shape
    return torch.cat([lv.reshape(B, N, -1, C) for lv in levels], dim=2).contiguous()


def unpack_levels(packed: torch.Tensor, shapes: Sequence[Sequence[int]]) -> list:
    """The packed [B,N,P,C] layout -> views [B,N,H_l,W_l,C]."""
    B, N, _, C = packed.shape
    out, off = [], 0
    for (h, w) in shapes:
        out.append(packed[:, :, off:off + h * w].reshape(B, N, h, w, C))
        off += h * w
    return out


def forward_levels(packed: torch.Tensor, shapes: Sequence[Sequence[int]], K: torch.Tensor, R: torch.Tensor,
                   t: torch.Tensor, bev_range: Sequence[float], X: int, Y: int, Z: int, *,
                   with_counts: bool = False, out: Optional[torch.Tensor] = None):
    """fbev_forward_levels on packed level features [B,N,P,C]; ``shapes`` lists (H_l, W_l),
    level 0 first.  Returns (out [B,C,X,Y] fp32, counts or None)."""
    if packed.dim() != 4:
        raise ValueError("packed features must be [B,N,P,C]")
    if packed.dtype not in _DTYPES:
        raise ValueError(f"unsupported feature dtype {packed.dtype}")
    if not packed.is_cuda or not packed.is_contiguous():
        raise ValueError("features must be a contiguous device tensor")
    B, N, P, C = packed.shape
    H, W = (int(v) for v in shapes[0])
    ratios = level_ratios(H, W, shapes)
    if P != sum(int(h) * int(w) for (h, w) in shapes):
        raise ValueError(f"packed pixel axis {P} does not match the level shapes {list(shapes)}")
    dev = packed.device
    _check_cams(K, R, t, B, N, dev)
    if out is None:
        out = torch.empty((B, C, X, Y), dtype=torch.float32, device=dev)
    else:
        _check_out("out", out, (B, C, X, Y), dev)
    counts = torch.empty((B, X, Y, Z), dtype=torch.uint8, device=dev) if with_counts else None
    lib = _lib.load()
    _lib.check(lib.fbev_forward_levels(_ptr(packed), _DTYPES[packed.dtype], _lib.feat_desc(B, N, C, H, W),
                                       len(ratios), _lib.int32_array(ratios), _ptr(K), _ptr(R), _ptr(t),
                                       _lib.bev_range(bev_range), X, Y, Z, _ptr(out), _ptr(counts), _stream(dev)))
    return out, counts


def backward_levels(grad_out: torch.Tensor, B: int, N: int, C: int, shapes: Sequence[Sequence[int]],
                    K: torch.Tensor, R: torch.Tensor, t: torch.Tensor, bev_range: Sequence[float],
                    X: int, Y: int, Z: int) -> torch.Tensor:
    """fbev_backward_levels: dL/dF as fp32 packed [B,N,P,C] from grad_out [B,C,X,Y]."""
    if tuple(grad_out.shape) != (B, C, X, Y) or grad_out.dtype != torch.float32:
        raise ValueError("grad_out must be float32 [B,C,X,Y]")
    grad_out = grad_out.contiguous()
    H, W = (int(v) for v in shapes[0])
    ratios = level_ratios(H, W, shapes)
    P = sum(int(h) * int(w) for (h, w) in shapes)
    _check_device_tensor("grad_out", grad_out)
    dev = grad_out.device
    _check_cams(K, R, t, B, N, dev)
    gF = torch.empty((B, N, P, C), dtype=torch.float32, device=dev)
    lib = _lib.load()
    _lib.check(lib.fbev_backward_levels(_ptr(grad_out), _lib.feat_desc(B, N, C, H, W), len(ratios),
                                        _lib.int32_array(ratios), _ptr(K), _ptr(R), _ptr(t),
                                        _lib.bev_range(bev_range), X, Y, Z, _ptr(gF), _stream(dev)))
    return gF


# ---- Lift-Splat (the push view transform)

def _check_lss_inputs(depth: torch.Tensor, context: torch.Tensor):
    if depth.dim() != 5 or context.dim() != 5:
        raise ValueError("depth must be [B,N,H,W,D] and context [B,N,H,W,C]")
    if depth.shape[:4] != context.shape[:4]:
        raise ValueError(f"depth {tuple(depth.shape)} and context {tuple(context.shape)} disagree on [B,N,H,W]")
    for name, x in (("depth", depth), ("context", context)):
        if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 device tensor")
    if depth.device != context.device:
        raise ValueError("depth and context must be on the same device")


def lss_forward(depth: torch.Tensor, context: torch.Tensor, K: torch.Tensor, R: torch.Tensor, t: torch.Tensor,
                bev_range: Sequence[float], X: int, Y: int, d_min: float, d_step: float, *,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fbev_lss_forward: depth alpha [B,N,H,W,D], context c [B,N,H,W,C] (fp32, channels-last);
    bin k at camera depth d_min + k d_step.  Returns the pillar sums [B,C,X,Y] fp32."""
    _check_lss_inputs(depth, context)
    B, N, H, W, D = depth.shape
    C = context.shape[-1]
    dev = depth.device
    _check_cams(K, R, t, B, N, dev)
    if out is None:
        out = torch.empty((B, C, X, Y), dtype=torch.float32, device=dev)
    else:
        _check_out("out", out, (B, C, X, Y), dev)
    lib = _lib.load()
    _lib.check(lib.fbev_lss_forward(_ptr(depth), _ptr(context), _lib.feat_desc(B, N, C, H, W), D, float(d_min),
                                    float(d_step), _ptr(K), _ptr(R), _ptr(t), _lib.bev_range(bev_range), X, Y,
                                    _ptr(out), _stream(dev)))
    return out


def lss_backward(grad_out: torch.Tensor, depth: torch.Tensor, context: torch.Tensor, K: torch.Tensor,
                 R: torch.Tensor, t: torch.Tensor, bev_range: Sequence[float], X: int, Y: int, d_min: float,
                 d_step: float, *, grad_depth: Optional[torch.Tensor] = None,
                 grad_context: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """fbev_lss_backward: (dL/ddepth [B,N,H,W,D], dL/dcontext [B,N,H,W,C]) from dL/dout [B,C,X,Y]."""
    _check_lss_inputs(depth, context)
    B, N, H, W, D = depth.shape
    C = context.shape[-1]
    dev = depth.device
    _check_cams(K, R, t, B, N, dev)
    if tuple(grad_out.shape) != (B, C, X, Y) or grad_out.dtype != torch.float32 or not grad_out.is_contiguous() \
            or grad_out.device != dev:
        raise ValueError(f"grad_out must be a contiguous float32 [{B},{C},{X},{Y}] tensor on {dev}")
    if grad_depth is None:
        grad_depth = torch.empty_like(depth)
    if grad_context is None:
        grad_context = torch.empty_like(context)
    for name, g, ref in (("grad_depth", grad_depth, depth), ("grad_context", grad_context, context)):
        if g.shape != ref.shape or g.dtype != torch.float32 or not g.is_contiguous() or g.device != dev:
            raise ValueError(f"{name} must be a contiguous float32 tensor shaped like its input")
    lib = _lib.load()
    _lib.check(lib.fbev_lss_backward(_ptr(grad_out), _ptr(depth), _ptr(context), _lib.feat_desc(B, N, C, H, W), D,
                                     float(d_min), float(d_step), _ptr(K), _ptr(R), _ptr(t),
                                     _lib.bev_range(bev_range), X, Y, _ptr(grad_depth), _ptr(grad_context),
                                     _stream(dev)))
    return grad_depth, grad_context


# ---- Deformable Aggregation (multi-camera deformable sampling)

def _check_deform(features, K, R, t, anchors, offsets, weights):
    if features.dim() != 5 or features.dtype != torch.float32 or not features.is_cuda or not features.is_contiguous():
        raise ValueError("features must be a contiguous float32 [B,N,H,W,C] device tensor")
    B, N, H, W, C = features.shape
    dev = features.device
    _check_cams(K, R, t, B, N, dev)
    if anchors.dim() != 3 or anchors.shape[0] != B or anchors.shape[2] != 3:
        raise ValueError(f"anchors must be [B,Q,3], got {tuple(anchors.shape)}")
    Q = anchors.shape[1]
    if offsets.dim() != 4 or tuple(offsets.shape[:2]) != (B, Q) or offsets.shape[3] != 3:
        raise ValueError(f"offsets must be [B,Q,Kp,3], got {tuple(offsets.shape)}")
    Kp = offsets.shape[2]
    if tuple(weights.shape) != (B, Q, N, Kp):
        raise ValueError(f"weights must be [{B},{Q},{N},{Kp}], got {tuple(weights.shape)}")
    for name, x in (("anchors", anchors), ("offsets", offsets), ("weights", weights)):
        if x.dtype != torch.float32 or not x.is_contiguous() or x.device != dev:
            raise ValueError(f"{name} must be a contiguous float32 tensor on {dev}")
    return B, N, H, W, C, Q, Kp, dev


def deform_forward(features: torch.Tensor, K: torch.Tensor, R: torch.Tensor, t: torch.Tensor, anchors: torch.Tensor,
                   offsets: torch.Tensor, weights: torch.Tensor, *, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fbev_deform_forward: features [B,N,H,W,C] fp32, anchors [B,Q,3], offsets [B,Q,Kp,3],
    weights [B,Q,N,Kp]; returns [B,Q,C] fp32."""
    B, N, H, W, C, Q, Kp, dev = _check_deform(features, K, R, t, anchors, offsets, weights)
    if out is None:
        out = torch.empty((B, Q, C), dtype=torch.float32, device=dev)
    else:
        _check_out("out", out, (B, Q, C), dev)
    lib = _lib.load()
    _lib.check(lib.fbev_deform_forward(_ptr(features), _lib.feat_desc(B, N, C, H, W), _ptr(K), _ptr(R), _ptr(t),
                                       _ptr(anchors), _ptr(offsets), _ptr(weights), Q, Kp, _ptr(out), _stream(dev)))
    return out


def deform_backward(grad_out: torch.Tensor, features: torch.Tensor, K: torch.Tensor, R: torch.Tensor,
                    t: torch.Tensor, anchors: torch.Tensor, offsets: torch.Tensor, weights: torch.Tensor, *,
                    with_anchors: bool = True, workspace: Optional[torch.Tensor] = None):
    """fbev_deform_backward: (dL/dfeatures, dL/dweights, dL/doffsets, dL/danchors or None).
    ``workspace`` (a uint8 device tensor) is allocated when not given or too small."""
    B, N, H, W, C, Q, Kp, dev = _check_deform(features, K, R, t, anchors, offsets, weights)
    if tuple(grad_out.shape) != (B, Q, C) or grad_out.dtype != torch.float32 or not grad_out.is_contiguous() \
            or grad_out.device != dev:
        raise ValueError(f"grad_out must be a contiguous float32 [{B},{Q},{C}] tensor on {dev}")
    gF = torch.empty_like(features)
    gW = torch.empty_like(weights)
    gO = torch.empty_like(offsets)
    gA = torch.empty_like(anchors) if with_anchors else None
    lib = _lib.load()
    fd = _lib.feat_desc(B, N, C, H, W)
    need = ctypes.c_size_t(0)
    _lib.check(lib.fbev_deform_backward_workspace(fd, Q, Kp, ctypes.byref(need)))
    if workspace is not None:
        _check_workspace(workspace, dev)
    if workspace is None or workspace.numel() < need.value:
        workspace = torch.empty((max(need.value, 1),), dtype=torch.uint8, device=dev)
    _lib.check(lib.fbev_deform_backward(_ptr(grad_out), _ptr(features), fd, _ptr(K), _ptr(R), _ptr(t),
                                        _ptr(anchors), _ptr(offsets), _ptr(weights), Q, Kp, _ptr(gF), _ptr(gW),
                                        _ptr(gO), _ptr(gA), _ptr(workspace), workspace.numel(), _stream(dev)))
    return gF, gW, gO, gA
