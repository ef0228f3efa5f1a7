"""CPU oracle for the temporal fused view transform (numpy, float64).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
module; only the tests, the smoke check and the benchmark's CPU-baseline leg
use it.  It shares no code with the HIP path.

What it computes.  The FlashBEV notes name a temporal fused view transform as
future work ("Takeaway" item 4); the pages give its two ingredients without a
formula: history must be brought into the current ego frame before it is
compared with the present, compensating the ego motion (SparseDriveV2 notes,
map and temporal sections, "ego-motion compensation"), and two BEV maps of
one scene are combined by stacking them in the same BEV space (Lift-Splat-
Shoot tutorial, the BEVFusion paragraph).  So, for batch sample b,

    out[b] = concat_channels( SamplingVT(F_t)[b],  align(prev_bev[b], A[b]) )

where align resamples the previous frame's BEV map at every current cell
centre mapped into the previous ego frame.

Readings taken where the pages leave a step open (listed in the design notes):
  T1  ego motion is a planar affine map A [B, 2, 3] from current-ego (x, y) to
      previous-ego (x', y'): [x'; y'] = A [x; y; 1] (a rigid motion in
      practice: rotation about z and a translation); heights play no part;
  T2  the previous map lives on the same grid (range, X, Y) as the current one
      and uses the cell-centre convention of the Sampling-VT: (x', y') sits at
      continuous index i' = (x' - x_min)/dx - 1/2, j' = (y' - y_min)/dy - 1/2;
  T3  it is sampled bilinearly inside the closed box [0, X-1] x [0, Y-1] of
      cell centres (the clamped tap at i' = X-1 has weight 0, as in S4) and is
      0 outside: a cell the previous grid did not cover has no history;
  T4  the two maps are stacked along channels, current first:
      out [B, C + Cp, X, Y];
  T5  backward: dL/dF from the first C channels (the Sampling-VT adjoint) and
      dL/dprev_bev = the adjoint of the resampling (each output cell's
      gradient goes to its four taps with their weights); no gradient with
      respect to the ego motion.
"""
from __future__ import annotations

from typing import Dict, Sequence

import numpy as np

from .sampling_vt import EDGE_EPS_PX, bilinear_taps, oracle_backward, oracle_forward


def cell_centres(rng6: Sequence[float], X: int, Y: int):
    """Metric centres of the current grid's cells: x [X], y [Y]."""
    xmin, xmax, ymin, ymax = (float(r) for r in rng6[:4])
    xs = xmin + (np.arange(X, dtype=np.float64) + 0.5) * ((xmax - xmin) / X)
    ys = ymin + (np.arange(Y, dtype=np.float64) + 0.5) * ((ymax - ymin) / Y)
    return xs, ys


def source_indices(A: np.ndarray, rng6: Sequence[float], X: int, Y: int):
    """Continuous indices (i', j') [X, Y] in the previous grid of every current cell centre (T1, T2)."""
    A = np.asarray(A, np.float64)
    xmin, xmax, ymin, ymax = (float(r) for r in rng6[:4])
    dx, dy = (xmax - xmin) / X, (ymax - ymin) / Y
    xs, ys = cell_centres(rng6, X, Y)
    gx, gy = np.meshgrid(xs, ys, indexing="ij")
    xp = A[0, 0] * gx + A[0, 1] * gy + A[0, 2]
    yp = A[1, 0] * gx + A[1, 1] * gy + A[1, 2]
    return (xp - xmin) / dx - 0.5, (yp - ymin) / dy - 0.5


def align_prev_bev(prev: np.ndarray, A: np.ndarray, rng6: Sequence[float]) -> Dict[str, np.ndarray]:
    """The previous BEV map [B, Cp, X, Y] resampled at the current cells (T1-T3).

    Returns ``aligned`` [B, Cp, X, Y], ``inside`` [B, X, Y] (the source is in
    the closed box) and ``near_border`` [B, X, Y] (the source within 1e-4 cells
    of the box's edges, where a rounding flip of the test changes the value).
    """
    prev = np.asarray(prev, np.float64)
    B, Cp, X, Y = prev.shape
    aligned = np.zeros_like(prev)
    inside = np.zeros((B, X, Y), bool)
    near = np.zeros((B, X, Y), bool)
    for b in range(B):
        si, sj = source_indices(A[b], rng6, X, Y)
        m = (si >= 0) & (si <= X - 1) & (sj >= 0) & (sj <= Y - 1)
        inside[b] = m
        e = EDGE_EPS_PX
        nearly = (si > -e) & (si < X - 1 + e) & (sj > -e) & (sj < Y - 1 + e)
        edge = (np.abs(si) < e) | (np.abs(si - (X - 1)) < e) | (np.abs(sj) < e) | (np.abs(sj - (Y - 1)) < e)
        near[b] = nearly & edge
        # the previous map indexed [i, j]: rows along x (size X), columns along y (size Y)
        for (ii, jj, w) in bilinear_taps(sj, si, m, X, Y):
            aligned[b] += prev[b][:, ii, jj] * w[None]
    return {"aligned": aligned, "inside": inside, "near_border": near}


def align_adjoint(g_aligned: np.ndarray, A: np.ndarray, rng6: Sequence[float]) -> np.ndarray:
    """Adjoint of ``align_prev_bev`` (T5): g [B, Cp, X, Y] -> dL/dprev [B, Cp, X, Y]."""
    g = np.asarray(g_aligned, np.float64)
    B, Cp, X, Y = g.shape
    out = np.zeros_like(g)
    for b in range(B):
        si, sj = source_indices(A[b], rng6, X, Y)
        m = (si >= 0) & (si <= X - 1) & (sj >= 0) & (sj <= Y - 1)
        for (ii, jj, w) in bilinear_taps(sj, si, m, X, Y):
            flat = (ii * Y + jj).ravel()
            contrib = (g[b] * w[None]).reshape(Cp, -1)
            for c in range(Cp):
                out[b, c] += np.bincount(flat, weights=contrib[c], minlength=X * Y).reshape(X, Y)
    return out


def temporal_forward(F, K, R, t, rng6, X: int, Y: int, Z: int, prev, A) -> Dict[str, np.ndarray]:
    """out [B, C + Cp, X, Y] = current Sampling-VT channels, then the aligned previous map (T4)."""
    cur = oracle_forward(F, K, R, t, rng6, X, Y, Z)
    al = align_prev_bev(prev, A, rng6)
    return {"out": np.concatenate([cur["out"], al["aligned"]], axis=1), "counts": cur["counts"],
            "near_edge": cur["near_edge"], "near_border": al["near_border"]}


def temporal_backward(grad_out, K, R, t, rng6, X: int, Y: int, Z: int, H: int, W: int, C: int, A):
    """(dL/dF [B, N, C, H, W], dL/dprev_bev [B, Cp, X, Y]) of ``temporal_forward`` (T5)."""
    g = np.asarray(grad_out, np.float64)
    if C == 0:                                  # no current channels: an empty feature gradient
        gF = np.zeros((g.shape[0], np.asarray(K).shape[1], 0, H, W), np.float64)
    else:
        gF = oracle_backward(g[:, :C], K, R, t, rng6, X, Y, Z, H, W)
    return gF, align_adjoint(g[:, C:], A, rng6)
