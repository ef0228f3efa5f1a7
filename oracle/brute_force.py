"""Scalar brute-force checker for the Sampling-VT oracle (pure Python, float64).

TEST INFRASTRUCTURE ONLY; it shares no code with ``sampling_vt`` (which it
checks) nor with the HIP path.

It evaluates one output element at a time the way the FlashBEV notes describe
the per-element gather-reduction ("Core Idea"; "Method" item 2): for cell
(b, i, j), for every height bin k and camera n, build the voxel centre,
transform it into the camera (p_cam = R p + t), apply K, divide by the depth,
test depth > 0 and the closed in-view box [0, W-1] x [0, H-1], interpolate the
four neighbouring pixels, average over the cameras that see the point, and add
the per-bin means over k.  Written with explicit loops and ``math`` only.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple


def _centre(lo: float, hi: float, n: int, i: int) -> float:
    return lo + (i + 0.5) * (hi - lo) / n


def _to_pixel(K, R, t, p) -> Tuple[float, float, float]:
    pc = [R[r][0] * p[0] + R[r][1] * p[1] + R[r][2] * p[2] + t[r] for r in range(3)]
    h = [K[r][0] * pc[0] + K[r][1] * pc[1] + K[r][2] * pc[2] for r in range(3)]
    d = h[2]
    if d == 0.0:
        return d, math.inf, math.inf
    return d, h[0] / d, h[1] / d


def _sample(img_c, H: int, W: int, u: float, v: float) -> float:
    """Bilinear value of one channel image ``img_c[y][x]`` at pixel-centre coords (u, v)."""
    xl = math.floor(u)
    yt = math.floor(v)
    fx = u - xl
    fy = v - yt
    xr = xl + 1 if xl + 1 < W else W - 1
    yb = yt + 1 if yt + 1 < H else H - 1
    top = img_c[yt][xl] * (1.0 - fx) + img_c[yt][xr] * fx
    bot = img_c[yb][xl] * (1.0 - fx) + img_c[yb][xr] * fx
    return top * (1.0 - fy) + bot * fy


def cell_value(F, K, R, t, rng6: Sequence[float], X: int, Y: int, Z: int,
               b: int, i: int, j: int) -> Tuple[List[float], List[int]]:
    """Output channels out[b, :, i, j] and the per-bin valid-camera counts.

    F is indexable as F[b][n][c][y][x]; K, R as [b][n][3][3]; t as [b][n][3].
    """
    N = len(F[b])
    C = len(F[b][0])
    H = len(F[b][0][0])
    W = len(F[b][0][0][0])
    xmin, xmax, ymin, ymax, zmin, zmax = (float(r) for r in rng6)
    px = _centre(xmin, xmax, X, i)
    py = _centre(ymin, ymax, Y, j)
    acc = [0.0] * C
    counts = []
    for k in range(Z):
        p = (px, py, _centre(zmin, zmax, Z, k))
        seen = []
        for n in range(N):
            d, u, v = _to_pixel(K[b][n], R[b][n], t[b][n], p)
            if d > 0.0 and 0.0 <= u <= W - 1 and 0.0 <= v <= H - 1:
                seen.append((n, u, v))
        counts.append(len(seen))
        if not seen:
            continue
        for c in range(C):
            s = 0.0
            for (n, u, v) in seen:
                s += _sample(F[b][n][c], H, W, u, v)
            acc[c] += s / len(seen)
    return acc, counts


def brute_forward(F, K, R, t, rng6, X: int, Y: int, Z: int):
    """Whole output [B][C][X][Y] and counts [B][X][Y][Z] as nested lists (tiny sizes only)."""
    B = len(F)
    C = len(F[0][0])
    out = [[[[0.0] * Y for _ in range(X)] for _ in range(C)] for _ in range(B)]
    cnt = [[[None] * Y for _ in range(X)] for _ in range(B)]
    for b in range(B):
        for i in range(X):
            for j in range(Y):
                vals, cs = cell_value(F, K, R, t, rng6, X, Y, Z, b, i, j)
                for c in range(C):
                    out[b][c][i][j] = vals[c]
                cnt[b][i][j] = cs
    return out, cnt


def cell_value_levels(levels, K, R, t, rng6: Sequence[float], X: int, Y: int, Z: int,
                      b: int, i: int, j: int) -> Tuple[List[float], List[int]]:
    """Multi-level variant of ``cell_value``: levels[l][b][n][c][y][x] are the
    maps of level l (level 0 the finest; its size is an integer multiple r_l of
    level l's).  A camera that sees the point at level 0 contributes the mean,
    over levels, of the bilinear value at u_l = (u + 1/2)/r_l - 1/2 (v likewise),
    each clamped into the level's pixel-centre box."""
    N = len(levels[0][b])
    C = len(levels[0][b][0])
    H0 = len(levels[0][b][0][0])
    W0 = len(levels[0][b][0][0][0])
    xmin, xmax, ymin, ymax, zmin, zmax = (float(r) for r in rng6)
    px = _centre(xmin, xmax, X, i)
    py = _centre(ymin, ymax, Y, j)
    acc = [0.0] * C
    counts = []
    for k in range(Z):
        p = (px, py, _centre(zmin, zmax, Z, k))
        seen = []
        for n in range(N):
            d, u, v = _to_pixel(K[b][n], R[b][n], t[b][n], p)
            if d > 0.0 and 0.0 <= u <= W0 - 1 and 0.0 <= v <= H0 - 1:
                seen.append((n, u, v))
        counts.append(len(seen))
        if not seen:
            continue
        for c in range(C):
            s = 0.0
            for (n, u, v) in seen:
                lv = 0.0
                for lev in levels:
                    H = len(lev[b][n][c])
                    W = len(lev[b][n][c][0])
                    r = H0 // H
                    ul = min(max((u + 0.5) / r - 0.5, 0.0), W - 1.0)
                    vl = min(max((v + 0.5) / r - 0.5, 0.0), H - 1.0)
                    lv += _sample(lev[b][n][c], H, W, ul, vl)
                s += lv / len(levels)
            acc[c] += s / len(seen)
    return acc, counts


def _inv3(M):
    """Inverse of a 3x3 matrix (nested lists) by cofactors."""
    a, b, c = M[0]
    d, e, f = M[1]
    g, h, i = M[2]
    co = [[e * i - f * h, -(d * i - f * g), d * h - e * g],
          [-(b * i - c * h), a * i - c * g, -(a * h - b * g)],
          [b * f - c * e, -(a * f - c * d), a * e - b * d]]
    det = a * co[0][0] + b * co[0][1] + c * co[0][2]
    return [[co[col][row] / det for col in range(3)] for row in range(3)]


def lss_brute(depth, context, K, R, t, rng6: Sequence[float], X: int, Y: int, d_min: float, d_step: float):
    """Lift-splat by scalar loops (Lift-Splat-Shoot tutorial, "Lift" and "Splat"): every
    pixel's D points along its ray (bin k at camera depth d_min + k d_step), each carrying
    depth[k] * context, moved to the ego frame and summed into its BEV cell.
    depth[b][n][k][v][u], context[b][n][c][v][u]; returns out[b][c][i][j] as nested lists."""
    B = len(depth)
    N = len(depth[0])
    D = len(depth[0][0])
    H = len(depth[0][0][0])
    W = len(depth[0][0][0][0])
    C = len(context[0][0])
    xmin, xmax, ymin, ymax = (float(r) for r in rng6[:4])
    dx = (xmax - xmin) / X
    dy = (ymax - ymin) / Y
    out = [[[[0.0] * Y for _ in range(X)] for _ in range(C)] for _ in range(B)]
    for b in range(B):
        for n in range(N):
            Ki = _inv3(K[b][n])
            Rn, tn = R[b][n], t[b][n]
            for v in range(H):
                for u in range(W):
                    ray = [Ki[r][0] * u + Ki[r][1] * v + Ki[r][2] for r in range(3)]
                    for k in range(D):
                        dep = d_min + k * d_step
                        pc = [dep * ray[r] - tn[r] for r in range(3)]
                        p = [Rn[0][r] * pc[0] + Rn[1][r] * pc[1] + Rn[2][r] * pc[2] for r in range(3)]
                        i = math.floor((p[0] - xmin) / dx)
                        j = math.floor((p[1] - ymin) / dy)
                        if 0 <= i < X and 0 <= j < Y:
                            a = depth[b][n][k][v][u]
                            for c in range(C):
                                out[b][c][i][j] += a * context[b][n][c][v][u]
    return out


def deform_brute(F, K, R, t, anchors, offsets, weights, b: int, q: int) -> List[float]:
    """Deformable Aggregation output out[b, q, :] by explicit loops (SparseDriveV2
    notes, "Deformable Aggregation", steps 1-3): keypoint = anchor + offset, each
    camera's projection, depth > 0 and the closed pixel-centre box, bilinear
    value times the (query, camera, keypoint) weight, summed.

    F is indexable as F[b][n][c][y][x]; anchors [b][q][3]; offsets [b][q][k][3];
    weights [b][q][n][k].
    """
    N = len(F[b])
    C = len(F[b][0])
    H = len(F[b][0][0])
    W = len(F[b][0][0][0])
    acc = [0.0] * C
    for k in range(len(offsets[b][q])):
        p = [anchors[b][q][r] + offsets[b][q][k][r] for r in range(3)]
        for n in range(N):
            d, u, v = _to_pixel(K[b][n], R[b][n], t[b][n], p)
            if not (d > 0.0 and 0.0 <= u <= W - 1 and 0.0 <= v <= H - 1):
                continue
            w = weights[b][q][n][k]
            for c in range(C):
                acc[c] += w * _sample(F[b][n][c], H, W, u, v)
    return acc


def align_brute(prev_b, A_b, rng6: Sequence[float], X: int, Y: int, c: int, i: int, j: int) -> float:
    """One element of the aligned previous BEV map: current cell (i, j) mapped into the previous
    ego frame by the planar affine A_b (2 x 3), then bilinear on the previous grid's cell centres,
    0 outside the closed box of centres.  ``prev_b`` is indexed [c][i][j]."""
    x = _centre(rng6[0], rng6[1], X, i)
    y = _centre(rng6[2], rng6[3], Y, j)
    xp = A_b[0][0] * x + A_b[0][1] * y + A_b[0][2]
    yp = A_b[1][0] * x + A_b[1][1] * y + A_b[1][2]
    si = (xp - rng6[0]) / ((rng6[1] - rng6[0]) / X) - 0.5
    sj = (yp - rng6[2]) / ((rng6[3] - rng6[2]) / Y) - 0.5
    if not (0.0 <= si <= X - 1 and 0.0 <= sj <= Y - 1):
        return 0.0
    i0, j0 = int(math.floor(si)), int(math.floor(sj))
    a, bb = si - i0, sj - j0
    i1, j1 = min(i0 + 1, X - 1), min(j0 + 1, Y - 1)
    p = prev_b[c]
    return ((1 - a) * (1 - bb) * p[i0][j0] + (1 - a) * bb * p[i0][j1] + a * (1 - bb) * p[i1][j0] + a * bb * p[i1][j1])
