"""CPU oracle for the exact dense Sampling-VT view transform (numpy, float64).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
module; only the tests, the smoke check and the benchmark's CPU-baseline leg
use it.  It shares no code with the HIP path.

What it computes (FlashBEV reading notes, "Problem Setting" and "Method"
items 1 and 4): the *tensorized* Sampling-VT pipeline, materialised stage by
stage exactly as the notes describe it,

    voxel grid -> projected coords -> mask -> sampled 3D features
               -> valid-camera mean (per height bin) -> height sum,

for every batch sample b.  The fused operator is claimed to reach this result
exactly, up to floating-point order ("Method" item 4), so this plain
definition is the parity target.

Readings taken where the pages leave a step open (each is listed with its
reason in the design notes):
  * voxel centres of half-open ranges: x_i = xmin + (i + 1/2)(xmax - xmin)/X,
    likewise y_j and z_k; out[b, c, i, j] has i along ego x and j along ego y;
  * projection  [u, v, 1]^T ~ K (R p + t)  with (R, t) ego->camera
    (SparseDriveV2 notes, "Deformable Aggregation" step 2): h = K (R p + t),
    d = h_3, u = h_1 / d, v = h_2 / d; integer (u, v) are pixel centres, u runs
    along W and v along H;
  * in view: d > 0 and 0 <= u <= W-1 and 0 <= v <= H-1 (closed, on pixel
    centres), so every valid sample is a convex combination of real pixels;
  * bilinear: x0 = floor(u), y0 = floor(v), a = u - x0, b = v - y0,
    x1 = min(x0 + 1, W - 1), y1 = min(y0 + 1, H - 1) (the clamped tap has
    weight exactly 0);
  * mean over the valid cameras of each (b, x, y, z) -- divide by the count,
    0 when no camera sees the point -- then the sum over z ("Method" item 1);
  * backward = gradient w.r.t. the features only; the map is linear in F with
    the mask, weights and counts fixed, so it is the exact adjoint.

Precision: every stage runs in float64; fp32 / bf16 inputs are widened
exactly.  Memory: the materialised stages are built for a block of X-rows at
a time (cells are independent, "Core Idea"), which changes no arithmetic.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

EDGE_EPS_PX = 1e-4
_MAX_CHUNK_ELEMS = 1 << 24   # elements of one materialised [N, C, rows, Y, Z] stage


def voxel_grid(rng6: Sequence[float], X: int, Y: int, Z: int, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Stage 1 ("voxel grid"): metric cell centres, shape [len(rows), Y, Z, 3].

    FlashBEV notes, "Problem Setting" (the tensorized form builds a voxel
    grid) and "Core Idea" (voxel construction is the first per-cell step).
    """
    xmin, xmax, ymin, ymax, zmin, zmax = (float(r) for r in rng6)
    if rows is None:
        rows = np.arange(X)
    xs = xmin + (np.asarray(rows, np.float64) + 0.5) * ((xmax - xmin) / X)
    ys = ymin + (np.arange(Y, dtype=np.float64) + 0.5) * ((ymax - ymin) / Y)
    zs = zmin + (np.arange(Z, dtype=np.float64) + 0.5) * ((zmax - zmin) / Z)
    g = np.empty((len(xs), Y, Z, 3), np.float64)
    g[..., 0] = xs[:, None, None]
    g[..., 1] = ys[None, :, None]
    g[..., 2] = zs[None, None, :]
    return g


def project(points: np.ndarray, K: np.ndarray, R: np.ndarray, t: np.ndarray):
    """Stage 2 ("projected coords"): depth d and pixel coords (u, v) per camera.

    SparseDriveV2 notes, "Deformable Aggregation" step 2:
    [u, v, 1]^T ~ K_i (R_i [X, Y, Z]^T + t_i).
    ``points`` is [..., 3] in the ego frame; K, R are [N,3,3], t is [N,3].
    Returns d, u, v, each [N, ...].
    """
    K = np.asarray(K, np.float64)
    R = np.asarray(R, np.float64)
    t = np.asarray(t, np.float64)
    p_cam = np.einsum("nij,...j->n...i", R, points) + t.reshape((t.shape[0],) + (1,) * (points.ndim - 1) + (3,))
    h = np.einsum("nij,n...j->n...i", K, p_cam)
    d = h[..., 2]
    with np.errstate(divide="ignore", invalid="ignore"):
        u = h[..., 0] / d
        v = h[..., 1] / d
    return d, u, v


def in_view_mask(d: np.ndarray, u: np.ndarray, v: np.ndarray, H: int, W: int) -> np.ndarray:
    """Stage 3 ("mask"): depth > 0 and (u, v) inside the closed pixel-centre box.

    FlashBEV notes, "Method" item 2 (validity check); the in-view rule of the
    SparseDriveV2 notes ("Deformable Aggregation" step 2), read on pixel
    centres as [0, W-1] x [0, H-1].
    """
    with np.errstate(invalid="ignore"):
        return (d > 0) & (u >= 0) & (u <= W - 1) & (v >= 0) & (v <= H - 1)


def near_edge_mask(d: np.ndarray, u: np.ndarray, v: np.ndarray, H: int, W: int, eps: float = EDGE_EPS_PX) -> np.ndarray:
    """Per (n, cell, z): a (nearly) in-view sample within ``eps`` px of an image edge.

    Counts at such points may legitimately differ between two correct
    implementations (a rounding flip of the in-view test), so parity
    comparisons exclude them.
    """
    with np.errstate(invalid="ignore"):
        nearly = (d > 0) & (u > -eps) & (u < W - 1 + eps) & (v > -eps) & (v < H - 1 + eps)
        edge = (np.abs(u) < eps) | (np.abs(u - (W - 1)) < eps) | (np.abs(v) < eps) | (np.abs(v - (H - 1)) < eps)
    return nearly & edge


def bilinear_taps(u: np.ndarray, v: np.ndarray, mask: np.ndarray, H: int, W: int):
    """Integer taps and weights of the bilinear interpolation at (u, v).

    Returns a list of four (y, x, w) triples; w is zero where ``mask`` is false
    (and the indices are then 0, a harmless in-range placeholder).
    FlashBEV notes, "Core Idea" / "Method" item 2 (bilinear sampling).
    """
    uu = np.where(mask, u, 0.0)
    vv = np.where(mask, v, 0.0)
    x0 = np.floor(uu)
    y0 = np.floor(vv)
    a = uu - x0
    b = vv - y0
    x0 = x0.astype(np.int64)
    y0 = y0.astype(np.int64)
    x1 = np.minimum(x0 + 1, W - 1)
    y1 = np.minimum(y0 + 1, H - 1)
    m = mask.astype(np.float64)
    return [
        (y0, x0, (1 - a) * (1 - b) * m),
        (y0, x1, a * (1 - b) * m),
        (y1, x0, (1 - a) * b * m),
        (y1, x1, a * b * m),
    ]


def bilinear_sample(F: np.ndarray, u: np.ndarray, v: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """Stage 4 ("sampled 3D features"): [N, C, ...]; invalid entries are 0.

    ``F`` is one sample's feature maps [N, C, H, W]; u, v, mask are [N, ...].
    """
    N, C, H, W = F.shape
    n_idx = np.arange(N).reshape((N,) + (1,) * (u.ndim - 1))
    out = np.zeros((N, C) + u.shape[1:], np.float64)
    for (yy, xx, w) in bilinear_taps(u, v, mask, H, W):
        g = F[n_idx, :, yy, xx]                        # [N, ..., C]
        out += np.moveaxis(g, -1, 1) * w[:, None]
    return out


def valid_camera_mean(samples: np.ndarray, mask: np.ndarray):
    """Stage 5: mean over the cameras valid at each (cell, z); 0 if none.

    FlashBEV notes, "Method" item 1: per height bin, a valid mean over the
    visible cameras.  Returns (m [C, ...], cnt [...] as int64).
    """
    cnt = mask.sum(axis=0)
    m = samples.sum(axis=0) / np.maximum(cnt, 1)[None]
    return m, cnt


def valid_mean_adjoint_scale(mask: np.ndarray) -> np.ndarray:
    """Factor the valid-camera mean applies to each camera's sample: mask / max(cnt, 1)."""
    cnt = mask.sum(axis=0)
    return mask / np.maximum(cnt, 1)[None]


def height_sum(m: np.ndarray) -> np.ndarray:
    """Stage 6: sum over the trailing height axis ("Method" item 1)."""
    return m.sum(axis=-1)


def _rows_per_chunk(N: int, C: int, Y: int, Z: int) -> int:
    return max(1, _MAX_CHUNK_ELEMS // max(1, N * max(C, 1) * Y * Z))


def _as_f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def oracle_forward(F: np.ndarray, K: np.ndarray, R: np.ndarray, t: np.ndarray, rng6: Sequence[float],
                   X: int, Y: int, Z: int, rows: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Tensorized forward over features F [B,N,C,H,W] (logical layout).

    Returns ``out`` [B,C,len(rows),Y] (float64), ``counts`` [B,len(rows),Y,Z]
    (uint8 valid-camera counts) and ``near_edge`` [B,len(rows),Y,Z] (bool).
    ``rows`` restricts the result to those X indices (all by default).
    """
    F = _as_f64(F)
    B, N, C, H, W = F.shape
    rows = np.arange(X) if rows is None else np.asarray(rows, np.int64)
    out = np.zeros((B, C, len(rows), Y), np.float64)
    counts = np.zeros((B, len(rows), Y, Z), np.uint8)
    near = np.zeros((B, len(rows), Y, Z), bool)
    step = _rows_per_chunk(N, C, Y, Z)
    for b in range(B):
        for s in range(0, len(rows), step):
            r = rows[s:s + step]
            grid = voxel_grid(rng6, X, Y, Z, r)                 # [r, Y, Z, 3]
            d, u, v = project(grid, K[b], R[b], t[b])           # [N, r, Y, Z]
            mask = in_view_mask(d, u, v, H, W)
            feats3d = bilinear_sample(F[b], u, v, mask)         # [N, C, r, Y, Z]
            m, cnt = valid_camera_mean(feats3d, mask)           # [C, r, Y, Z]
            out[b, :, s:s + len(r)] = height_sum(m)
            counts[b, s:s + len(r)] = cnt.astype(np.uint8)
            near[b, s:s + len(r)] = near_edge_mask(d, u, v, H, W).any(axis=0)
    return {"out": out, "counts": counts, "near_edge": near}


def oracle_backward(grad_out: np.ndarray, K: np.ndarray, R: np.ndarray, t: np.ndarray, rng6: Sequence[float],
                    X: int, Y: int, Z: int, H: int, W: int, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Gradient of the forward w.r.t. the features, [B,N,C,H,W] float64.

    The forward is linear in F once the mask, bilinear weights and counts are
    fixed, so its gradient is the adjoint of each materialised stage taken in
    reverse order (FlashBEV notes, "Method" item 4, forward/backward
    equivalence):
      height sum   -> broadcast grad over z;
      valid mean   -> multiply by mask / max(cnt, 1);
      bilinear     -> scatter-add weight * value onto the four taps.
    """
    grad_out = _as_f64(grad_out)
    B, C = grad_out.shape[:2]
    N = K.shape[1]
    gF = np.zeros((B, N, C, H, W), np.float64)
    step = _rows_per_chunk(N, C, Y, Z)
    all_rows = np.arange(X) if rows is None else np.asarray(rows, np.int64)
    for b in range(B):
        acc = np.zeros((C, N * H * W), np.float64)
        for s in range(0, len(all_rows), step):
            r = all_rows[s:s + step]
            grid = voxel_grid(rng6, X, Y, Z, r)
            d, u, v = project(grid, K[b], R[b], t[b])
            mask = in_view_mask(d, u, v, H, W)
            g_m = np.broadcast_to(grad_out[b][:, r][:, :, :, None], (C, len(r), Y, Z))         # adjoint of height sum
            scale = valid_mean_adjoint_scale(mask)                                           # adjoint of valid mean
            g_s = g_m[None] * scale[:, None]                                                 # [N, C, r, Y, Z]
            n_idx = np.arange(N).reshape(N, 1, 1, 1)
            for (yy, xx, w) in bilinear_taps(u, v, mask, H, W):                              # adjoint of bilinear
                pix = (n_idx * (H * W) + yy * W + xx).ravel()
                contrib = (g_s * w[:, None]).transpose(1, 0, 2, 3, 4).reshape(C, -1)
                for c in range(C):
                    acc[c] += np.bincount(pix, weights=contrib[c], minlength=N * H * W)
        gF[b] = acc.reshape(C, N, H, W).transpose(1, 0, 2, 3)
    return gF


def tensorized_intermediates(F: np.ndarray, K: np.ndarray, R: np.ndarray, t: np.ndarray, rng6: Sequence[float],
                             X: int, Y: int, Z: int, b: int = 0) -> Dict[str, np.ndarray]:
    """Every materialised stage for one sample (small sizes only; for tests)."""
    F = _as_f64(F)
    _, N, C, H, W = F.shape
    grid = voxel_grid(rng6, X, Y, Z)
    d, u, v = project(grid, K[b], R[b], t[b])
    mask = in_view_mask(d, u, v, H, W)
    feats3d = bilinear_sample(F[b], u, v, mask)
    m, cnt = valid_camera_mean(feats3d, mask)
    return {"grid": grid, "d": d, "u": u, "v": v, "mask": mask, "features3d": feats3d,
            "mean": m, "cnt": cnt, "out": height_sum(m)}
