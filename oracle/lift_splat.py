"""CPU oracle for Lift-Splat (the push view transform), numpy float64.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
module; only the tests, the smoke check and the benchmark's CPU-baseline leg
use it.  It shares no code with the HIP path.

What it computes (Lift-Splat-Shoot tutorial, sections "Lift" and "Splat"):
every feature-map pixel of every camera predicts a distribution alpha over D
depth bins (softmax outside this operator) and a context vector c; "lift"
places D points along the pixel's ray, point d carrying alpha_d * c (the
outer product alpha (x) c); "splat" moves the points into the ego frame with
the camera's intrinsics and extrinsics and sums the features of all points
that fall into the same BEV cell, whatever their height (a pillar); the sum
is order-free over points and cameras.  Written as the plain definition:
compute every point, find its cell, add (``np.add.at``).

Readings taken where the pages leave a step open (listed in the design
notes):
  * depth bin k sits at depth d_k = d_min + k * d_step, k = 0 .. D-1 (the
    tutorial's nuScenes setting lists 4, 5, ..., 44 for the range [4, 45) at
    1 m); depth is the camera-frame z, so a pixel's point at depth d is
    p_cam = d K^-1 [u, v, 1]^T with integer (u, v) at pixel centres;
  * ego position p = R^T (p_cam - t), with (R, t) mapping ego to camera as
    in the pull transform;
  * BEV cell (i, j) = (floor((x - x_min) / dx), floor((y - y_min) / dy)) for
    x in [x_min, x_max), y in [y_min, y_max); points outside are dropped; no
    bound on height (one pillar per cell);
  * the backward is the exact adjoint with the geometry fixed:
    dL/dc = sum_d alpha_d g[cell_d], dL/dalpha_d = <c, g[cell_d]>.

Layouts: depth [B,N,D,H,W] and context [B,N,C,H,W] (logical); output
[B,C,X,Y].
"""
from __future__ import annotations

from typing import Dict, Sequence, Tuple

import numpy as np

EDGE_EPS_M = 1e-9   # points this close to a cell edge may fall either side in another correct implementation


def depth_values(d_min: float, d_step: float, D: int) -> np.ndarray:
    """Depth of each bin: d_min + k d_step (tutorial, "Lift": bins over [4, 45) at 1 m are 4, 5, ..., 44)."""
    return d_min + np.arange(D, dtype=np.float64) * d_step


def frustum_points(K: np.ndarray, R: np.ndarray, t: np.ndarray, H: int, W: int, depths: np.ndarray) -> np.ndarray:
    """Ego-frame points [N, D, H, W, 3] of every camera's pixels at every bin depth.

    Tutorial, "Splat" step 1: the lifted points sit on the pixels' rays in the
    camera frame and are moved to the ego frame with the intrinsics and
    extrinsics (the inverse of the pull transform's projection).
    """
    K = np.asarray(K, np.float64)
    R = np.asarray(R, np.float64)
    t = np.asarray(t, np.float64)
    vs, us = np.meshgrid(np.arange(H, dtype=np.float64), np.arange(W, dtype=np.float64), indexing="ij")
    pix = np.stack([us, vs, np.ones_like(us)], axis=-1)                      # [H, W, 3]
    rays = np.einsum("nij,hwj->nhwi", np.linalg.inv(K), pix)                 # K^-1 [u, v, 1]: z_cam = 1
    p_cam = depths[None, :, None, None, None] * rays[:, None]                 # [N, D, H, W, 3]
    return np.einsum("nji,ndhwj->ndhwi", R, p_cam - t[:, None, None, None, :])   # R^T (p_cam - t)


def bev_cells(points: np.ndarray, rng6: Sequence[float], X: int, Y: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Cell indices (i, j) of ego points and the in-grid mask (tutorial, "Splat" step 2)."""
    xmin, xmax, ymin, ymax = (float(r) for r in rng6[:4])
    dx = (xmax - xmin) / X
    dy = (ymax - ymin) / Y
    i = np.floor((points[..., 0] - xmin) / dx)
    j = np.floor((points[..., 1] - ymin) / dy)
    inside = (i >= 0) & (i < X) & (j >= 0) & (j < Y)
    return np.where(inside, i, 0).astype(np.int64), np.where(inside, j, 0).astype(np.int64), inside


def near_cell_edge(points: np.ndarray, rng6: Sequence[float], X: int, Y: int, eps: float = EDGE_EPS_M) -> np.ndarray:
    """Points within ``eps`` metres of a cell edge (their cell is a rounding decision)."""
    xmin, xmax, ymin, ymax = (float(r) for r in rng6[:4])
    fx = (points[..., 0] - xmin) / ((xmax - xmin) / X)
    fy = (points[..., 1] - ymin) / ((ymax - ymin) / Y)
    dx = np.abs(fx - np.round(fx)) * ((xmax - xmin) / X)
    dy = np.abs(fy - np.round(fy)) * ((ymax - ymin) / Y)
    return (dx < eps) | (dy < eps)


def lss_forward(depth: np.ndarray, context: np.ndarray, K: np.ndarray, R: np.ndarray, t: np.ndarray,
                rng6: Sequence[float], X: int, Y: int, d_min: float, d_step: float) -> Dict[str, np.ndarray]:
    """Lift-splat forward: ``out`` [B,C,X,Y] float64 and ``near_edge`` [B,N,D,H,W] (bool).

    ``depth`` is [B,N,D,H,W] (a distribution over bins per pixel), ``context`` [B,N,C,H,W].
    """
    depth = np.asarray(depth, np.float64)
    context = np.asarray(context, np.float64)
    B, N, D, H, W = depth.shape
    C = context.shape[2]
    zs = depth_values(d_min, d_step, D)
    out = np.zeros((B, C, X, Y), np.float64)
    near = np.zeros((B, N, D, H, W), bool)
    for b in range(B):
        pts = frustum_points(K[b], R[b], t[b], H, W, zs)                     # [N, D, H, W, 3]
        i, j, inside = bev_cells(pts, rng6, X, Y)
        near[b] = near_cell_edge(pts, rng6, X, Y) & inside
        # lift: point (n, d, v, u) carries alpha[n, d, v, u] * c[n, :, v, u]   (the outer product)
        lifted = depth[b][:, :, None] * context[b][:, None]                  # [N, D, C, H, W]
        flat = (i * Y + j)[inside]                                           # [P] cell of each kept point
        feats = np.moveaxis(lifted, 2, -1)[inside]                           # [P, C]
        acc = np.zeros((X * Y, C), np.float64)
        np.add.at(acc, flat, feats)                                          # splat: sum per cell
        out[b] = acc.T.reshape(C, X, Y)
    return {"out": out, "near_edge": near}


def lss_backward(grad_out: np.ndarray, depth: np.ndarray, context: np.ndarray, K: np.ndarray, R: np.ndarray,
                 t: np.ndarray, rng6: Sequence[float], X: int, Y: int, d_min: float,
                 d_step: float) -> Tuple[np.ndarray, np.ndarray]:
    """Adjoint of ``lss_forward``: (dL/ddepth [B,N,D,H,W], dL/dcontext [B,N,C,H,W]), float64.

    With the geometry fixed the forward is bilinear in (alpha, c): each kept
    point contributes alpha_d c to its cell, so dL/dalpha_d = <c, g[cell]> and
    dL/dc = sum over the pixel's kept points of alpha_d g[cell].
    """
    grad_out = np.asarray(grad_out, np.float64)
    depth = np.asarray(depth, np.float64)
    context = np.asarray(context, np.float64)
    B, N, D, H, W = depth.shape
    C = context.shape[2]
    zs = depth_values(d_min, d_step, D)
    g_depth = np.zeros_like(depth)
    g_ctx = np.zeros_like(context)
    for b in range(B):
        pts = frustum_points(K[b], R[b], t[b], H, W, zs)
        i, j, inside = bev_cells(pts, rng6, X, Y)
        g_pts = np.where(inside[..., None], grad_out[b][:, i, j].transpose(1, 2, 3, 4, 0), 0.0)   # [N, D, H, W, C]
        c_pts = np.moveaxis(context[b], 1, -1)[:, None]                                           # [N, 1, H, W, C]
        g_depth[b] = (g_pts * c_pts).sum(axis=-1)
        g_ctx[b] = np.moveaxis((g_pts * depth[b][..., None]).sum(axis=1), -1, 1)
    return g_depth, g_ctx
