"""CPU oracle for the multi-level (feature-pyramid) Sampling-VT (numpy, float64).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
module; only the tests, the smoke check and the benchmark's CPU-baseline leg
use it.  It shares no code with the HIP path.

The pages name a multi-scale fused view transform as the natural next step
(FlashBEV reading notes, "Limitation" item 4: multi-scale features are among
the deployment conditions the evaluation leaves open; "Takeaway" item 4:
multi-scale / temporal fused VT as future work) and describe the pyramid it
would read (SparseDriveV2 notes, "Multi-scale features": FPN outputs P2-P5 at
growing strides, fine levels for small or distant objects, coarse levels for
large or near ones).  No page defines the fused operator itself, so this
module fixes the plainest reading that keeps the single-level operator as its
L = 1 case:

  * each camera has L feature maps; level l is H_l x W_l with
    H_0 = r_l H_l and W_0 = r_l W_l for an integer ratio r_l >= 1 (r_0 = 1);
    K maps to level-0 pixels;
  * validity and the valid-camera count are the single-level rule at level 0
    (depth > 0 and (u, v) in the closed box [0, W_0-1] x [0, H_0-1]): a camera
    sees the point or not, whatever the level;
  * level l is sampled at the same image point.  A level-l pixel centre sits
    at the centre of the r_l x r_l block of level-0 pixels it covers, so the
    level coordinate is u_l = (u + 1/2) / r_l - 1/2 (v likewise), clamped to
    the level's pixel-centre box [0, W_l-1] x [0, H_l-1] (border replication:
    a constant map samples to that constant at every level);
  * a camera's sample is the mean of its L level samples; the valid-camera
    mean over cameras and the sum over height bins follow as in the
    single-level operator ("Method" item 1 of the FlashBEV notes).

Features are given per level as [B, N, C, H_l, W_l] (logical layout).
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

from .sampling_vt import (bilinear_sample, bilinear_taps, height_sum, in_view_mask, near_edge_mask, project,
                          valid_camera_mean, valid_mean_adjoint_scale, voxel_grid)

_MAX_CHUNK_ELEMS = 1 << 24


def level_ratios(shapes: Sequence[Sequence[int]]) -> List[int]:
    """Integer ratios r_l = H_0 / H_l = W_0 / W_l of level shapes [(H_l, W_l), ...]."""
    H0, W0 = shapes[0]
    ratios = []
    for (H, W) in shapes:
        if H <= 0 or W <= 0 or H0 % H or W0 % W or H0 // H != W0 // W:
            raise ValueError(f"level {H}x{W} is not an integer downscale of {H0}x{W0}")
        ratios.append(H0 // H)
    return ratios


def level_coords(u: np.ndarray, v: np.ndarray, r: int, H: int, W: int):
    """Level-r pixel coordinates of level-0 point (u, v), clamped to the level's box."""
    ul = (u + 0.5) / r - 0.5
    vl = (v + 0.5) / r - 0.5
    return np.clip(ul, 0.0, W - 1.0), np.clip(vl, 0.0, H - 1.0)


def multilevel_sample(levels: Sequence[np.ndarray], b: int, u: np.ndarray, v: np.ndarray,
                      mask: np.ndarray, ratios: Sequence[int]) -> np.ndarray:
    """Per-camera sample [N, C, ...]: the mean over levels of each level's bilinear sample."""
    out = None
    for F, r in zip(levels, ratios):
        H, W = F.shape[-2:]
        ul, vl = level_coords(np.where(mask, u, 0.0), np.where(mask, v, 0.0), r, H, W)
        s = bilinear_sample(np.asarray(F[b], np.float64), ul, vl, mask)
        out = s if out is None else out + s
    return out / len(levels)


def _rows_per_chunk(N: int, C: int, Y: int, Z: int) -> int:
    return max(1, _MAX_CHUNK_ELEMS // max(1, N * max(C, 1) * Y * Z))


def oracle_forward_levels(levels: Sequence[np.ndarray], K: np.ndarray, R: np.ndarray, t: np.ndarray,
                          rng6: Sequence[float], X: int, Y: int, Z: int,
                          rows: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Forward over per-level features [B,N,C,H_l,W_l]; same outputs as ``oracle_forward``."""
    B, N, C, H0, W0 = levels[0].shape
    ratios = level_ratios([F.shape[-2:] for F in levels])
    rows = np.arange(X) if rows is None else np.asarray(rows, np.int64)
    out = np.zeros((B, C, len(rows), Y), np.float64)
    counts = np.zeros((B, len(rows), Y, Z), np.uint8)
    near = np.zeros((B, len(rows), Y, Z), bool)
    step = _rows_per_chunk(N, C, Y, Z)
    for b in range(B):
        for s in range(0, len(rows), step):
            r = rows[s:s + step]
            grid = voxel_grid(rng6, X, Y, Z, r)
            d, u, v = project(grid, K[b], R[b], t[b])
            mask = in_view_mask(d, u, v, H0, W0)
            feats3d = multilevel_sample(levels, b, u, v, mask, ratios)     # [N, C, r, Y, Z]
            m, cnt = valid_camera_mean(feats3d, mask)
            out[b, :, s:s + len(r)] = height_sum(m)
            counts[b, s:s + len(r)] = cnt.astype(np.uint8)
            near[b, s:s + len(r)] = near_edge_mask(d, u, v, H0, W0).any(axis=0)
    return {"out": out, "counts": counts, "near_edge": near}


def oracle_backward_levels(grad_out: np.ndarray, K: np.ndarray, R: np.ndarray, t: np.ndarray,
                           rng6: Sequence[float], X: int, Y: int, Z: int,
                           shapes: Sequence[Sequence[int]], rows: Optional[Sequence[int]] = None) -> List[np.ndarray]:
    """Gradient w.r.t. each level's features, a list of [B,N,C,H_l,W_l] float64
    (only the cells of X-rows ``rows`` contribute when given).

    The adjoint of each stage in reverse order: the height sum broadcasts the
    gradient over z, the valid mean multiplies by mask / max(cnt, 1), the level
    mean by 1 / L, and each level's bilinear sample scatters weight * value onto
    its four taps.
    """
    grad_out = np.asarray(grad_out, np.float64)
    B, C = grad_out.shape[:2]
    N = K.shape[1]
    H0, W0 = shapes[0]
    ratios = level_ratios(shapes)
    L = len(shapes)
    grads = [np.zeros((B, N, C, H, W), np.float64) for (H, W) in shapes]
    step = _rows_per_chunk(N, C, Y, Z)
    n_idx = np.arange(N).reshape(N, 1, 1, 1)
    for b in range(B):
        accs = [np.zeros((C, N * H * W), np.float64) for (H, W) in shapes]
        all_rows = np.arange(X) if rows is None else np.asarray(rows, np.int64)
        for s in range(0, len(all_rows), step):
            r = all_rows[s:s + step]
            grid = voxel_grid(rng6, X, Y, Z, r)
            d, u, v = project(grid, K[b], R[b], t[b])
            mask = in_view_mask(d, u, v, H0, W0)
            g_m = np.broadcast_to(grad_out[b][:, r][:, :, :, None], (C, len(r), Y, Z))
            g_s = g_m[None] * valid_mean_adjoint_scale(mask)[:, None] / L          # [N, C, r, Y, Z]
            for li, ((H, W), rl) in enumerate(zip(shapes, ratios)):
                ul, vl = level_coords(np.where(mask, u, 0.0), np.where(mask, v, 0.0), rl, H, W)
                for (yy, xx, w) in bilinear_taps(ul, vl, mask, H, W):
                    pix = (n_idx * (H * W) + yy * W + xx).ravel()
                    contrib = (g_s * w[:, None]).transpose(1, 0, 2, 3, 4).reshape(C, -1)
                    for c in range(C):
                        accs[li][c] += np.bincount(pix, weights=contrib[c], minlength=N * H * W)
        for li, (H, W) in enumerate(shapes):
            grads[li][b] = accs[li].reshape(C, N, H, W).transpose(1, 0, 2, 3)
    return grads
