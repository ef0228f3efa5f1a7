"""CPU oracle for fused Deformable Aggregation (multi-camera deformable
sampling, the operator a fused spatial cross-attention is built on), numpy
float64.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
module; only the tests, the smoke check and the benchmark's CPU-baseline leg
use it.  It shares no code with the HIP path.

What it computes (SparseDriveV2 notes, "Deformable Aggregation", steps 1-3;
the FlashBEV notes carry the same fusion over to BEVFormer's spatial
cross-attention): every query q of batch sample b has a 3D anchor a_q and K
keypoint offsets Delta_{q,k}, and

  step 1   p_{q,k} = a_q + Delta_{q,k}                              (ego frame, metres)
  step 2   per camera i:  [u, v, 1]^T ~ K_i (R_i p + t_i),  in view or not
  step 3   out_q = sum_i sum_k  w_{q,i,k} * in_view * bilinear(F_i, u, v)

Readings taken where the pages leave a step open (listed in the design notes):
  D1  the sampling function is the bilinear sample; its "small neighbourhood"
      is the four taps, and the predicted weights w are the attention;
  D2  in view: depth > 0 and (u, v) in the closed box of pixel centres
      [0, W-1] x [0, H-1].  The page's box [0, W] x [0, H] is the image extent
      in edge coordinates; with integer (u, v) at pixel centres (the
      convention of the rest of this library) the closed centre box keeps
      every sample a convex combination of real pixels;
  D3  weights are given per (query, camera, keypoint), [B, Q, N, K], and are
      used as written: out-of-view pairs contribute nothing and nothing is
      renormalised;
  D4  anchors [B, Q, 3] and offsets [B, Q, K, 3] in the ego frame;
  D5  backward: with respect to the features (the adjoint scatter), the
      weights (dw = in_view * <sample, g>) and the keypoint positions (the
      chain rule through the projection and the bilinear interpolation,
      which is bilinear in (u, v) inside a pixel square), so that
      dL/dDelta_{q,k} = dL/dp_{q,k} and dL/da_q = sum_k dL/dp_{q,k}.

Layouts: features [B, N, C, H, W] (logical), output [B, Q, C].
"""
from __future__ import annotations

from typing import Dict, Tuple

import numpy as np

from .sampling_vt import bilinear_sample, bilinear_taps, in_view_mask, near_edge_mask, project


def keypoints(anchors: np.ndarray, offsets: np.ndarray) -> np.ndarray:
    """Step 1: p_{q,k} = a_q + Delta_{q,k}, [Q, K, 3] for one batch sample."""
    return np.asarray(anchors, np.float64)[:, None, :] + np.asarray(offsets, np.float64)


def deform_forward(F: np.ndarray, K: np.ndarray, R: np.ndarray, t: np.ndarray, anchors: np.ndarray,
                   offsets: np.ndarray, weights: np.ndarray) -> Dict[str, np.ndarray]:
    """Forward: ``out`` [B, Q, C] float64, ``valid`` [B, N, Q, K] and ``near_edge`` [B, N, Q, K] (bool)."""
    F = np.asarray(F, np.float64)
    weights = np.asarray(weights, np.float64)
    B, N, C, H, W = F.shape
    Q, Kp = offsets.shape[1:3]
    out = np.zeros((B, Q, C), np.float64)
    valid = np.zeros((B, N, Q, Kp), bool)
    near = np.zeros((B, N, Q, Kp), bool)
    for b in range(B):
        pts = keypoints(anchors[b], offsets[b])                          # [Q, K, 3]
        d, u, v = project(pts, K[b], R[b], t[b])                         # [N, Q, K]
        m = in_view_mask(d, u, v, H, W)
        valid[b] = m
        near[b] = near_edge_mask(d, u, v, H, W)
        s = bilinear_sample(F[b], u, v, m)                               # [N, C, Q, K]
        w = np.moveaxis(weights[b], 1, 0) * m                            # [N, Q, K]
        out[b] = np.einsum("ncqk,nqk->qc", s, w)                         # step 3: sum over cameras and keypoints
    return {"out": out, "valid": valid, "near_edge": near}


def _sample_gradients(Fb: np.ndarray, u: np.ndarray, v: np.ndarray, m: np.ndarray):
    """Derivatives of the bilinear sample with respect to u and v, [N, C, ...] each.

    Inside the pixel square the sample is (1-a)(1-b) F00 + a(1-b) F01 + (1-a) b F10 + a b F11
    with a = u - x0, b = v - y0, so d/du = (1-b)(F01 - F00) + b(F11 - F10) and
    d/dv = (1-a)(F10 - F00) + a(F11 - F01).
    """
    N, C, H, W = Fb.shape
    uu = np.where(m, u, 0.0)
    vv = np.where(m, v, 0.0)
    x0 = np.floor(uu)
    y0 = np.floor(vv)
    a = uu - x0
    bb = vv - y0
    x0 = x0.astype(np.int64)
    y0 = y0.astype(np.int64)
    x1 = np.minimum(x0 + 1, W - 1)
    y1 = np.minimum(y0 + 1, H - 1)
    n_idx = np.arange(N).reshape((N,) + (1,) * (u.ndim - 1))

    def tap(yy, xx):
        return np.moveaxis(Fb[n_idx, :, yy, xx], -1, 1)                  # [N, C, ...]

    F00, F01, F10, F11 = tap(y0, x0), tap(y0, x1), tap(y1, x0), tap(y1, x1)
    mm = m[:, None].astype(np.float64)
    a = a[:, None]
    bb = bb[:, None]
    du = ((1 - bb) * (F01 - F00) + bb * (F11 - F10)) * mm
    dv = ((1 - a) * (F10 - F00) + a * (F11 - F01)) * mm
    return du, dv


def _projection_jacobian(pts: np.ndarray, K: np.ndarray, R: np.ndarray, t: np.ndarray):
    """d(u, v)/dp for every camera and point: two arrays [N, ..., 3].

    h = M p + c with M = K R and c = K t; u = h_1 / h_3, v = h_2 / h_3, so
    du/dp = (M_1 - u M_3) / h_3 and dv/dp = (M_2 - v M_3) / h_3 (rows M_i).
    """
    K = np.asarray(K, np.float64)
    R = np.asarray(R, np.float64)
    t = np.asarray(t, np.float64)
    M = np.einsum("nij,njk->nik", K, R)                                  # [N, 3, 3]
    c = np.einsum("nij,nj->ni", K, t)                                    # [N, 3]
    h = np.einsum("nij,...j->n...i", M, pts) + c.reshape((c.shape[0],) + (1,) * (pts.ndim - 1) + (3,))
    with np.errstate(divide="ignore", invalid="ignore"):
        u = h[..., 0] / h[..., 2]
        v = h[..., 1] / h[..., 2]
        shape = (M.shape[0],) + (1,) * (pts.ndim - 1) + (3,)
        du = (M[:, 0, :].reshape(shape) - u[..., None] * M[:, 2, :].reshape(shape)) / h[..., 2:3]
        dv = (M[:, 1, :].reshape(shape) - v[..., None] * M[:, 2, :].reshape(shape)) / h[..., 2:3]
    return du, dv


def deform_backward(grad_out: np.ndarray, F: np.ndarray, K: np.ndarray, R: np.ndarray, t: np.ndarray,
                    anchors: np.ndarray, offsets: np.ndarray, weights: np.ndarray
                    ) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """Adjoint of ``deform_forward``: (dL/dF [B,N,C,H,W], dL/dw [B,Q,N,K], dL/doffsets [B,Q,K,3],
    dL/danchors [B,Q,3]), float64; the in-view mask is held fixed."""
    g = np.asarray(grad_out, np.float64)
    F = np.asarray(F, np.float64)
    weights = np.asarray(weights, np.float64)
    B, N, C, H, W = F.shape
    Q, Kp = offsets.shape[1:3]
    gF = np.zeros_like(F)
    gw = np.zeros((B, Q, N, Kp), np.float64)
    gp = np.zeros((B, Q, Kp, 3), np.float64)
    n_idx = np.arange(N).reshape(N, 1, 1)
    for b in range(B):
        pts = keypoints(anchors[b], offsets[b])
        d, u, v = project(pts, K[b], R[b], t[b])
        m = in_view_mask(d, u, v, H, W)
        w = np.moveaxis(weights[b], 1, 0) * m                            # [N, Q, K]
        gq = g[b].T                                                      # [C, Q]
        # features: each in-view sample scatters w * tap weight * g onto its four taps
        acc = np.zeros((C, N * H * W), np.float64)
        for (yy, xx, tw) in bilinear_taps(u, v, m, H, W):
            pix = (n_idx * (H * W) + yy * W + xx).ravel()
            contrib = (gq[:, None, :, None] * (w * tw)[None]).reshape(C, -1)   # [C, N*Q*K]
            for c in range(C):
                acc[c] += np.bincount(pix, weights=contrib[c], minlength=N * H * W)
        gF[b] = acc.reshape(C, N, H, W).transpose(1, 0, 2, 3)
        # weights: the sample's dot product with the upstream gradient
        s = bilinear_sample(F[b], u, v, m)                               # [N, C, Q, K]
        gw[b] = np.moveaxis(np.einsum("ncqk,cq->nqk", s, gq) * m, 0, 1)
        # keypoints: chain rule through the bilinear sample and the projection
        su, sv = _sample_gradients(F[b], u, v, m)                        # [N, C, Q, K]
        lu = np.einsum("ncqk,cq->nqk", su, gq) * w                       # dL/du per (camera, query, keypoint)
        lv = np.einsum("ncqk,cq->nqk", sv, gq) * w
        ju, jv = _projection_jacobian(pts, K[b], R[b], t[b])             # [N, Q, K, 3]
        gp[b] = np.nansum(np.where(m[..., None], lu[..., None] * ju + lv[..., None] * jv, 0.0), axis=0)
    return gF, gw, gp, gp.sum(axis=2)
