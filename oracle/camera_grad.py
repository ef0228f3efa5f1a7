"""CPU oracle for the gradients of the dense Sampling-VT output with respect to
the camera parameters K, R and t (numpy, float64).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
module; only the tests, the smoke check and the benchmark's CPU-baseline leg
use it.  It shares no code with the HIP path.

What it computes.  The SparseDriveV2 notes ("Deformable Aggregation",
pitfalls) ask that the sampling stay differentiable so that gradients flow
through the whole projection-and-sampling chain; the FlashBEV notes' Sampling
VT ("Method" items 1-4) is such a chain from the cameras to the BEV output.
For an upstream gradient g [B, C, X, Y] and L = <g, out>, this module returns
dL/dK [B,N,3,3], dL/dR [B,N,3,3] and dL/dt [B,N,3] of the tensorized forward
in `oracle.sampling_vt`.

Readings taken where the pages leave a step open (listed in the design notes):
  G1  the in-view mask and the valid-camera counts are held fixed: both are
      piecewise constant in the cameras, so their derivative is zero wherever
      it exists, and the derivative is that of the remaining smooth map;
  G2  inside the pixel square that floor() selects, the bilinear sample is
      bilinear in (u, v); its partial derivatives are those of that square
      (one-sided on the square's left and top edges);
  G3  K, R and t are free arrays: every entry gets its partial derivative (no
      orthonormality constraint on R; the fixed zeros and the one of K get
      theirs too);
  G4  the chain is taken through P = K [R | t]: with p~ = (x, y, z, 1) and
      h = P p~, u = h_1 / h_3 and v = h_2 / h_3, so
          du/dP_1j = p~_j / h_3,   du/dP_3j = -u p~_j / h_3,
          dv/dP_2j = p~_j / h_3,   dv/dP_3j = -v p~_j / h_3,
      and dL/dK = dL/dP [R | t]^T, dL/d[R | t] = K^T dL/dP.

Per in-view sample (b, cell, height bin, camera) the upstream gradient of
that camera's sample is g[b, :, cell] / count (the valid-camera mean and the
height sum, "Method" item 1), so dL/du is that vector's dot product with
d(sample)/du over the channels, and likewise for v.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from .deform_agg import _sample_gradients as sample_uv_derivatives
from .sampling_vt import in_view_mask, near_edge_mask, project, valid_mean_adjoint_scale, voxel_grid

_MAX_CHUNK_ELEMS = 1 << 22   # elements of one materialised [N, C, rows, Y, Z] derivative


def pixel_gradients(grad_out_b: np.ndarray, Fb: np.ndarray, u: np.ndarray, v: np.ndarray, mask: np.ndarray,
                    rows: np.ndarray):
    """dL/du and dL/dv per (camera, cell, bin) of one batch sample, [N, r, Y, Z] each.

    ``grad_out_b`` is g[b] [C, X, Y]; u, v, mask are [N, r, Y, Z] for the X-rows ``rows``.
    """
    su, sv = sample_uv_derivatives(Fb, u, v, mask)                     # [N, C, r, Y, Z]
    gc = grad_out_b[:, rows]                                             # [C, r, Y]
    scale = valid_mean_adjoint_scale(mask)                               # mask / max(count, 1)
    lu = np.einsum("ncryz,cry->nryz", su, gc) * scale
    lv = np.einsum("ncryz,cry->nryz", sv, gc) * scale
    return lu, lv


def projection_gradient(lu: np.ndarray, lv: np.ndarray, d: np.ndarray, u: np.ndarray, v: np.ndarray,
                        mask: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """dL/dP [N, 3, 4] from dL/du, dL/dv at every sample (reading G4)."""
    pt = np.concatenate([grid, np.ones(grid.shape[:-1] + (1,))], axis=-1)    # [r, Y, Z, 4]
    with np.errstate(divide="ignore", invalid="ignore"):
        a = np.where(mask, lu / d, 0.0)
        b = np.where(mask, lv / d, 0.0)
        c = np.where(mask, -(lu * u + lv * v) / d, 0.0)
    gP = np.empty((lu.shape[0], 3, 4), np.float64)
    gP[:, 0] = np.einsum("nryz,ryzj->nj", a, pt)
    gP[:, 1] = np.einsum("nryz,ryzj->nj", b, pt)
    gP[:, 2] = np.einsum("nryz,ryzj->nj", c, pt)
    return gP


def oracle_camera_backward(grad_out: np.ndarray, F: np.ndarray, K: np.ndarray, R: np.ndarray, t: np.ndarray,
                           rng6: Sequence[float], X: int, Y: int, Z: int,
                           rows: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Gradients of L = <grad_out, out> with respect to the cameras.

    F is [B,N,C,H,W] (logical layout), grad_out [B,C,X,Y].  ``rows``
    restricts the sum to those X-rows (the exact gradient when grad_out is
    zero on every other row).  Returns ``K`` [B,N,3,3], ``R`` [B,N,3,3],
    ``t`` [B,N,3], ``P`` [B,N,3,4] (dL/dP) and ``near_edge`` [B,X,Y] (a
    cell with a sample within 1e-4 px of an image edge), all float64.
    """
    F = np.asarray(F, np.float64)
    g = np.asarray(grad_out, np.float64)
    K = np.asarray(K, np.float64)
    R = np.asarray(R, np.float64)
    t = np.asarray(t, np.float64)
    B, N, C, H, W = F.shape
    all_rows = np.arange(X) if rows is None else np.asarray(rows, np.int64)
    gP = np.zeros((B, N, 3, 4), np.float64)
    near = np.zeros((B, X, Y), bool)
    step = max(1, _MAX_CHUNK_ELEMS // max(1, N * max(C, 1) * Y * max(Z, 1)))
    for b in range(B):
        for s in range(0, len(all_rows), step):
            r = all_rows[s:s + step]
            grid = voxel_grid(rng6, X, Y, Z, r)                              # [r, Y, Z, 3]
            d, u, v = project(grid, K[b], R[b], t[b])                        # [N, r, Y, Z]
            mask = in_view_mask(d, u, v, H, W)
            near[b, r] = near_edge_mask(d, u, v, H, W).any(axis=(0, 3))
            if N == 0 or C == 0:
                continue
            lu, lv = pixel_gradients(g[b], F[b], u, v, mask, r)
            gP[b] += projection_gradient(lu, lv, d, u, v, mask, grid)
    M = np.concatenate([R, t[..., None]], axis=-1)                           # [B, N, 3, 4] = [R | t]
    gK = np.einsum("bnij,bnkj->bnik", gP, M)                                 # dL/dP [R | t]^T
    gM = np.einsum("bnki,bnkj->bnij", K, gP)                                 # K^T dL/dP
    return {"K": gK, "R": gM[..., :3], "t": gM[..., 3], "P": gP, "near_edge": near}
