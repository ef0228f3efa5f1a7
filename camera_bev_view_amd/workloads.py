"""Seeded synthetic inputs for the Sampling-VT view transform.

This module only *draws* inputs: camera rigs (K, R, t), feature maps,
upstream gradients and BEV ranges.  It holds none of the operator's own
arithmetic (no voxel centres, projection, validity test, sampling or
reduction), so both the CPU oracle and the GPU path can be fed from it
without sharing any of the computation under test.

The shapes follow the camera-BEV setting the FlashBEV reading notes
describe (B x N x C x H x W features, a B x C x X x Y output, Z height
bins; "Problem Setting"), with nuScenes-like sizes taken from the
Lift-Splat-Shoot tutorial (six surround cameras, an 8 x 22 stride-16
feature map, a +-50 m BEV at 0.5 m; "Lift" and "Splat" sections).  No
dataset is read: every tensor is drawn from a seeded numpy generator.

Rig convention (also used by the oracle's documentation):
  * ego frame: x forward, y left, z up (metres);
  * camera frame: x right, y down, z forward;
  * (R, t) maps ego to camera, p_cam = R p_ego + t, as in the projection
    equation of the SparseDriveV2 notes ("Deformable Aggregation", step 2);
  * camera k looks outward at yaw psi_k = k * 360/N deg + U(-5, 5) deg
    (counter-clockwise from +x seen from above), pitch 0, roll 0, with its
    centre 1 m from the ego origin along psi_k at height 1.6 m;
  * intrinsics are in feature-map pixels: fx = fy = (W/2) / tan(35 deg),
    cx = (W-1)/2, cy = (H-1)/2, so integer (u, v) are pixel centres.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import numpy as np

# Half of the horizontal field of view (70 deg in total).
HALF_HFOV_DEG = 35.0
CAM_RADIUS_M = 1.0
CAM_HEIGHT_M = 1.6
YAW_JITTER_DEG = 5.0


@dataclasses.dataclass(frozen=True)
class Workload:
    """One named problem size.  ``rng6`` = (xmin, xmax, ymin, ymax, zmin, zmax)."""

    cid: int
    name: str
    B: int
    N: int
    C: int
    H: int
    W: int
    X: int
    Y: int
    Z: int
    rng6: Tuple[float, float, float, float, float, float]
    dtypes: Tuple[str, ...]
    per_sample_rig: bool
    backward: bool

    @property
    def out_elems(self) -> int:
        return self.B * self.C * self.X * self.Y

    @property
    def tuples(self) -> int:
        return self.B * self.X * self.Y * self.Z * self.N


_R50 = (-50.0, 50.0, -50.0, 50.0, -5.0, 3.0)
_R512 = (-51.2, 51.2, -51.2, 51.2, -5.0, 3.0)

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload(0, "tiny", 1, 6, 16, 8, 22, 50, 50, 4, _R50, ("f32",), False, False),
    "nuscenes": Workload(1, "nuscenes", 1, 6, 64, 16, 44, 200, 200, 8, _R50, ("f32",), False, False),
    "batched": Workload(2, "batched", 4, 6, 80, 32, 88, 200, 200, 16, _R50, ("f32", "bf16"), True, False),
    "large": Workload(3, "large", 1, 6, 128, 64, 176, 400, 400, 32, _R50, ("bf16",), False, False),
    "fwdbwd": Workload(4, "fwdbwd", 2, 6, 64, 16, 44, 256, 256, 16, _R512, ("f32",), True, True),
}


def intrinsics(H: int, W: int) -> np.ndarray:
    """3x3 pinhole intrinsics in feature-map pixels (fp32)."""
    f = (W / 2.0) / math.tan(math.radians(HALF_HFOV_DEG))
    K = np.array([[f, 0.0, (W - 1) / 2.0], [0.0, f, (H - 1) / 2.0], [0.0, 0.0, 1.0]], dtype=np.float64)
    return K.astype(np.float32)


def extrinsics_from_yaw(yaw_deg: float, radius: float = CAM_RADIUS_M, height: float = CAM_HEIGHT_M,
                        pitch_deg: float = 0.0) -> Tuple[np.ndarray, np.ndarray]:
    """Ego->camera (R, t) for an outward-looking camera at ``yaw_deg``.

    Rows of R are the camera axes written in the ego frame:
    right = (sin psi, -cos psi, 0), down = (0, 0, -1), forward = (cos psi, sin psi, 0)
    for pitch 0.  A positive ``pitch_deg`` tilts the optical axis upward
    (rotation about the camera's right axis).  t = -R c with c the camera
    centre at ``radius`` along psi and ``height`` above the ego origin.
    """
    psi = math.radians(yaw_deg)
    th = math.radians(pitch_deg)
    right = np.array([math.sin(psi), -math.cos(psi), 0.0])
    fwd0 = np.array([math.cos(psi), math.sin(psi), 0.0])
    up0 = np.array([0.0, 0.0, 1.0])
    fwd = math.cos(th) * fwd0 + math.sin(th) * up0
    down = -(math.cos(th) * up0 - math.sin(th) * fwd0)
    R = np.stack([right, down, fwd])
    c = np.array([radius * math.cos(psi), radius * math.sin(psi), height])
    t = -R @ c
    return R.astype(np.float32), t.astype(np.float32)


def make_rig(cid: int, B: int, N: int, H: int, W: int, per_sample: bool,
             jitter: bool = True, pitch_deg: float = 0.0) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Seeded ring rig: K [B,N,3,3], R [B,N,3,3], t [B,N,3], all fp32.

    Sample b draws its yaw jitter from ``default_rng([cid, b, 0])`` when
    ``per_sample`` is set; otherwise every sample reuses the b = 0 rig.
    ``pitch_deg`` tilts every camera's optical axis upward by that angle.
    """
    K = np.empty((B, N, 3, 3), np.float32)
    R = np.empty((B, N, 3, 3), np.float32)
    t = np.empty((B, N, 3), np.float32)
    Kn = intrinsics(H, W)
    for b in range(B):
        g = np.random.default_rng([cid, b if per_sample else 0, 0])
        jit = g.uniform(-YAW_JITTER_DEG, YAW_JITTER_DEG, N) if jitter else np.zeros(N)
        for n in range(N):
            Rn, tn = extrinsics_from_yaw(n * 360.0 / N + float(jit[n]), pitch_deg=pitch_deg)
            K[b, n], R[b, n], t[b, n] = Kn, Rn, tn
    return K, R, t


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16 (round-to-nearest-even), returned as uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    nan = np.isnan(a)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to fp32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def make_features(cid: int, B: int, N: int, C: int, H: int, W: int, dtype: str = "f32") -> np.ndarray:
    """Logical [B,N,C,H,W] features ~ N(0,1) from ``default_rng([cid, 1])``.

    For ``dtype == "bf16"`` the fp32 draws are rounded to bfloat16 (RNE) and
    returned as their exact fp32 values, so every consumer sees the same
    numbers.
    """
    g = np.random.default_rng([cid, 1])
    F = g.standard_normal((B, N, C, H, W), dtype=np.float32)
    if dtype == "bf16":
        F = bf16_bits_to_f32(to_bf16_bits(F))
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return F


def make_grad_out(cid: int, B: int, C: int, X: int, Y: int) -> np.ndarray:
    """Upstream gradient [B,C,X,Y] ~ N(0,1) from ``default_rng([cid, 2])``."""
    g = np.random.default_rng([cid, 2])
    return g.standard_normal((B, C, X, Y), dtype=np.float32)


@dataclasses.dataclass
class Inputs:
    F: np.ndarray            # logical [B,N,C,H,W] fp32 values (bf16-representable when dtype == "bf16")
    K: np.ndarray
    R: np.ndarray
    t: np.ndarray
    rng6: Tuple[float, ...]
    X: int
    Y: int
    Z: int
    dtype: str
    grad_out: Optional[np.ndarray] = None


def make_inputs(name: str, dtype: Optional[str] = None, with_grad: bool = False, **override) -> Inputs:
    """Inputs for a named workload; keyword overrides replace its sizes (same seeds)."""
    w = dataclasses.replace(WORKLOADS[name], **override) if override else WORKLOADS[name]
    dt = dtype or w.dtypes[0]
    K, R, t = make_rig(w.cid, w.B, w.N, w.H, w.W, w.per_sample_rig)
    F = make_features(w.cid, w.B, w.N, w.C, w.H, w.W, dt)
    g = make_grad_out(w.cid, w.B, w.C, w.X, w.Y) if (with_grad or w.backward) else None
    return Inputs(F, K, R, t, tuple(float(np.float32(r)) for r in w.rng6), w.X, w.Y, w.Z, dt, g)


def random_case(seed: int, B: int, N: int, C: int, H: int, W: int, X: int, Y: int, Z: int,
                rng6=(-50.0, 50.0, -50.0, 50.0, -5.0, 3.0), dtype: str = "f32",
                per_sample: bool = True, with_grad: bool = True) -> Inputs:
    """An arbitrary-size seeded case (used for ragged / edge-case parity runs)."""
    K, R, t = make_rig(1000 + seed, B, N, H, W, per_sample)
    F = make_features(1000 + seed, B, N, C, H, W, dtype)
    g = make_grad_out(1000 + seed, B, C, X, Y) if with_grad else None
    return Inputs(F, K, R, t, tuple(float(np.float32(r)) for r in rng6), X, Y, Z, dtype, g)


# ---- feature pyramids (multi-level inputs)
#
# The pyramid stands in for FPN outputs at growing strides (the SparseDriveV2
# notes' "Multi-scale features": P2-P5).  Level 0 is the finest map; level l
# is smaller by an integer ratio r_l in both directions, and K is in level-0
# pixels.  The nuScenes-shaped pyramid takes strides 8, 16 and 32 of a
# 256 x 704 image: 32 x 88, 16 x 44 and 8 x 22 maps.

PYRAMIDS: Dict[str, dict] = {
    "pyramid": dict(cid=5, B=1, N=6, C=64, H=32, W=88, ratios=(1, 2, 4), X=200, Y=200, Z=8, rng6=_R50,
                    dtype="f32", per_sample=False),
}


def make_level_features(cid: int, B: int, N: int, C: int, shapes, dtype: str = "f32"):
    """Logical per-level features [B,N,C,H_l,W_l] ~ N(0,1); level l from ``default_rng([cid, 1, l])``."""
    out = []
    for l, (H, W) in enumerate(shapes):
        g = np.random.default_rng([cid, 1, l])
        F = g.standard_normal((B, N, C, H, W), dtype=np.float32)
        if dtype == "bf16":
            F = bf16_bits_to_f32(to_bf16_bits(F))
        elif dtype != "f32":
            raise ValueError(f"unknown dtype {dtype!r}")
        out.append(F)
    return out


@dataclasses.dataclass
class LevelInputs:
    levels: list             # logical [B,N,C,H_l,W_l] per level
    shapes: Tuple[Tuple[int, int], ...]
    K: np.ndarray            # [B,N,3,3] in level-0 pixels
    R: np.ndarray
    t: np.ndarray
    rng6: Tuple[float, ...]
    X: int
    Y: int
    Z: int
    dtype: str
    grad_out: Optional[np.ndarray] = None


def level_shapes(H: int, W: int, ratios) -> Tuple[Tuple[int, int], ...]:
    return tuple((H // r, W // r) for r in ratios)


def make_level_inputs(name: str = "pyramid", dtype: Optional[str] = None, with_grad: bool = False) -> LevelInputs:
    w = PYRAMIDS[name]
    dt = dtype or w["dtype"]
    shapes = level_shapes(w["H"], w["W"], w["ratios"])
    K, R, t = make_rig(w["cid"], w["B"], w["N"], w["H"], w["W"], w["per_sample"])
    levels = make_level_features(w["cid"], w["B"], w["N"], w["C"], shapes, dt)
    g = make_grad_out(w["cid"], w["B"], w["C"], w["X"], w["Y"]) if with_grad else None
    return LevelInputs(levels, shapes, K, R, t, tuple(float(np.float32(r)) for r in w["rng6"]), w["X"], w["Y"],
                       w["Z"], dt, g)


def random_level_case(seed: int, B: int, N: int, C: int, H: int, W: int, ratios, X: int, Y: int, Z: int,
                      rng6=(-50.0, 50.0, -50.0, 50.0, -5.0, 3.0), dtype: str = "f32") -> LevelInputs:
    """An arbitrary-size seeded pyramid case (ragged / edge-case parity runs)."""
    shapes = level_shapes(H, W, ratios)
    K, R, t = make_rig(2000 + seed, B, N, H, W, True)
    levels = make_level_features(2000 + seed, B, N, C, shapes, dtype)
    g = make_grad_out(2000 + seed, B, C, X, Y)
    return LevelInputs(levels, shapes, K, R, t, tuple(float(np.float32(r)) for r in rng6), X, Y, Z, dtype, g)


# ---- Lift-Splat (push view transform) inputs
#
# Sizes from the Lift-Splat-Shoot tutorial ("Lift" and "Splat"): six cameras,
# an 8 x 22 feature map (a 128 x 352 image at stride 16), C = 64 context
# channels, D = 41 depth bins over [4, 45) m at 1 m, and a 200 x 200 BEV grid
# of 0.5 m cells over +-50 m.  The batched workload doubles the map (a 256 x
# 704 image at stride 16) at batch 4 for throughput.  The depth distribution
# of each pixel is a draw from a flat Dirichlet (a point on the probability
# simplex, like the softmax output it stands for); the context is N(0, 1).

LSS_WORKLOADS: Dict[str, dict] = {
    "lss": dict(cid=6, B=1, N=6, C=64, H=8, W=22, D=41, d_min=4.0, d_step=1.0, X=200, Y=200, rng6=_R50,
                per_sample=False),
    "lss_batched": dict(cid=7, B=4, N=6, C=64, H=16, W=44, D=41, d_min=4.0, d_step=1.0, X=200, Y=200, rng6=_R50,
                        per_sample=True),
}


def make_depth_dist(cid: int, B: int, N: int, D: int, H: int, W: int) -> np.ndarray:
    """Logical depth distributions [B,N,D,H,W] fp32 from ``default_rng([cid, 3])`` (flat Dirichlet per pixel)."""
    g = np.random.default_rng([cid, 3])
    a = g.dirichlet(np.ones(max(D, 1)), size=(B, N, H, W))[..., :D] if D > 0 else np.zeros((B, N, H, W, 0))
    return np.ascontiguousarray(a.astype(np.float32).transpose(0, 1, 4, 2, 3))


@dataclasses.dataclass
class LssInputs:
    depth: np.ndarray        # logical [B,N,D,H,W] fp32
    context: np.ndarray      # logical [B,N,C,H,W] fp32
    K: np.ndarray
    R: np.ndarray
    t: np.ndarray
    rng6: Tuple[float, ...]
    X: int
    Y: int
    d_min: float
    d_step: float
    grad_out: Optional[np.ndarray] = None


def make_lss_inputs(name: str = "lss", with_grad: bool = False, **override) -> LssInputs:
    """Inputs for a named Lift-Splat workload; keyword overrides replace its sizes (same seeds)."""
    w = dict(LSS_WORKLOADS[name], **override)
    K, R, t = make_rig(w["cid"], w["B"], w["N"], w["H"], w["W"], w["per_sample"])
    depth = make_depth_dist(w["cid"], w["B"], w["N"], w["D"], w["H"], w["W"])
    ctx = make_features(w["cid"], w["B"], w["N"], w["C"], w["H"], w["W"])
    g = make_grad_out(w["cid"], w["B"], w["C"], w["X"], w["Y"]) if with_grad else None
    return LssInputs(depth, ctx, K, R, t, tuple(float(np.float32(r)) for r in w["rng6"]), w["X"], w["Y"],
                     float(np.float32(w["d_min"])), float(np.float32(w["d_step"])), g)


def random_lss_case(seed: int, B: int, N: int, C: int, H: int, W: int, D: int, X: int, Y: int,
                    rng6=(-50.0, 50.0, -50.0, 50.0, -5.0, 3.0), d_min: float = 4.0, d_step: float = 1.0,
                    pitch_deg: float = 0.0) -> LssInputs:
    """An arbitrary-size seeded Lift-Splat case (ragged / edge-case parity runs)."""
    K, R, t = make_rig(3000 + seed, B, N, H, W, True, pitch_deg=pitch_deg)
    depth = make_depth_dist(3000 + seed, B, N, D, H, W)
    ctx = make_features(3000 + seed, B, N, C, H, W)
    g = make_grad_out(3000 + seed, B, C, X, Y)
    return LssInputs(depth, ctx, K, R, t, tuple(float(np.float32(r)) for r in rng6), X, Y,
                     float(np.float32(d_min)), float(np.float32(d_step)), g)


# ---- Deformable Aggregation inputs
#
# The SparseDriveV2 notes give the operator's scale: queries ~10^2 with tens
# of keypoints each over up to six cameras (about 1.5 of them seeing a
# keypoint).  "deform" stands in for a sparse detection head: 900 queries,
# 13 keypoints, C = 256 on 16 x 44 maps (a 256 x 704 image at stride 16);
# anchors uniform over +-50 m at heights in [-1, 2] m, offsets N(0, 1 m) per
# axis.  "deform_bev" is the dense BEV form (spatial cross-attention over a
# 200 x 200 grid): one query per cell centre at z = 0, 8 keypoints at the
# height-bin centres of [-5, 3) m plus N(0, 0.1 m) jitter, C = 64.  Weights
# per query are a flat-Dirichlet draw over its (camera, keypoint) pairs (a
# point on the simplex, standing in for the network's softmax).

DEFORM_WORKLOADS: Dict[str, dict] = {
    "deform": dict(cid=8, B=1, N=6, C=256, H=16, W=44, Q=900, Kp=13, kind="sparse"),
    "deform_bev": dict(cid=9, B=1, N=6, C=64, H=16, W=44, X=200, Y=200, Kp=8, rng6=_R50, kind="bev"),
}


@dataclasses.dataclass
class DeformInputs:
    F: np.ndarray            # logical [B,N,C,H,W] fp32
    K: np.ndarray
    R: np.ndarray
    t: np.ndarray
    anchors: np.ndarray      # [B,Q,3] fp32
    offsets: np.ndarray      # [B,Q,Kp,3] fp32
    weights: np.ndarray      # [B,Q,N,Kp] fp32
    grad_out: Optional[np.ndarray] = None   # [B,Q,C] fp32


def _dirichlet_weights(g, B: int, Q: int, N: int, Kp: int) -> np.ndarray:
    if N * Kp == 0:
        return np.zeros((B, Q, N, Kp), np.float32)
    return g.dirichlet(np.ones(N * Kp), size=(B, Q)).reshape(B, Q, N, Kp).astype(np.float32)


def make_deform_inputs(name: str = "deform", with_grad: bool = False) -> DeformInputs:
    w = DEFORM_WORKLOADS[name]
    B, N, C, H, W, Kp, cid = w["B"], w["N"], w["C"], w["H"], w["W"], w["Kp"], w["cid"]
    K, R, t = make_rig(cid, B, N, H, W, False)
    F = make_features(cid, B, N, C, H, W)
    g = np.random.default_rng([cid, 4])
    if w["kind"] == "sparse":
        Q = w["Q"]
        anchors = np.stack([g.uniform(-50, 50, (B, Q)), g.uniform(-50, 50, (B, Q)), g.uniform(-1, 2, (B, Q))], -1)
        offsets = g.normal(0.0, 1.0, (B, Q, Kp, 3))
    else:
        X, Y = w["X"], w["Y"]
        xmin, xmax, ymin, ymax, zmin, zmax = w["rng6"]
        xs = xmin + (np.arange(X) + 0.5) * (xmax - xmin) / X
        ys = ymin + (np.arange(Y) + 0.5) * (ymax - ymin) / Y
        zs = zmin + (np.arange(Kp) + 0.5) * (zmax - zmin) / Kp
        Q = X * Y
        anchors = np.zeros((B, Q, 3))
        anchors[..., 0] = np.repeat(xs, Y)[None]
        anchors[..., 1] = np.tile(ys, X)[None]
        offsets = g.normal(0.0, 0.1, (B, Q, Kp, 3))
        offsets[..., 2] += zs[None, None, :]
    weights = _dirichlet_weights(g, B, Q, N, Kp)
    gout = np.random.default_rng([cid, 2]).standard_normal((B, Q, C), dtype=np.float32) if with_grad else None
    return DeformInputs(F, K, R, t, anchors.astype(np.float32), offsets.astype(np.float32), weights, gout)


def random_deform_case(seed: int, B: int, N: int, C: int, H: int, W: int, Q: int, Kp: int, spread: float = 30.0,
                       offset_sigma: float = 1.5, pitch_deg: float = 0.0) -> DeformInputs:
    """An arbitrary-size seeded Deformable Aggregation case (ragged / edge-case parity runs)."""
    K, R, t = make_rig(4000 + seed, B, N, H, W, True, pitch_deg=pitch_deg)
    F = make_features(4000 + seed, B, N, C, H, W)
    g = np.random.default_rng([4000 + seed, 4])
    anchors = np.stack([g.uniform(-spread, spread, (B, Q)), g.uniform(-spread, spread, (B, Q)),
                        g.uniform(-1, 2, (B, Q))], -1)
    offsets = g.normal(0.0, offset_sigma, (B, Q, Kp, 3))
    weights = _dirichlet_weights(g, B, Q, N, Kp)
    gout = np.random.default_rng([4000 + seed, 2]).standard_normal((B, Q, C), dtype=np.float32)
    return DeformInputs(F, K, R, t, anchors.astype(np.float32), offsets.astype(np.float32), weights, gout)


# ---- temporal fusion inputs
#
# The previous frame's BEV map stands in for the output of the previous step:
# N(0, 1) values on the current grid.  The ego motion maps current-ego (x, y)
# to previous-ego (x, y): a yaw of U(-5, 5) degrees and a move of U(2, 8) m
# forward and U(-0.5, 0.5) m sideways per sample, the motion of a car between
# frames half a second apart, from ``default_rng([id, 5])``.

TEMPORAL_WORKLOADS: Dict[str, dict] = {
    "temporal": dict(base="nuscenes", cid=10, Cp=64),
}


def make_ego_motion(cid: int, B: int, yaw_deg: Optional[float] = None, shift=None) -> np.ndarray:
    """[B, 2, 3] fp32 planar motions current-ego (x, y) -> previous-ego (x, y)."""
    g = np.random.default_rng([cid, 5])
    A = np.empty((B, 2, 3), np.float64)
    for b in range(B):
        psi = math.radians(g.uniform(-5.0, 5.0) if yaw_deg is None else yaw_deg)
        tx, ty = (g.uniform(2.0, 8.0), g.uniform(-0.5, 0.5)) if shift is None else shift
        A[b] = [[math.cos(psi), -math.sin(psi), tx], [math.sin(psi), math.cos(psi), ty]]
    return A.astype(np.float32)


@dataclasses.dataclass
class TemporalInputs:
    cur: Inputs
    prev: np.ndarray          # [B, Cp, X, Y] fp32
    ego: np.ndarray           # [B, 2, 3] fp32
    grad_out: np.ndarray      # [B, C + Cp, X, Y] fp32


def make_temporal_inputs(name: str = "temporal") -> TemporalInputs:
    w = TEMPORAL_WORKLOADS[name]
    cur = make_inputs(w["base"], with_grad=False)
    B, C = cur.F.shape[0], cur.F.shape[2]
    prev = np.random.default_rng([w["cid"], 1]).standard_normal((B, w["Cp"], cur.X, cur.Y), dtype=np.float32)
    g = np.random.default_rng([w["cid"], 2]).standard_normal((B, C + w["Cp"], cur.X, cur.Y), dtype=np.float32)
    return TemporalInputs(cur, prev, make_ego_motion(w["cid"], B), g)


def random_temporal_case(seed: int, B: int, N: int, C: int, H: int, W: int, X: int, Y: int, Z: int, Cp: int,
                         rng6=(-30.0, 30.0, -30.0, 30.0, -4.0, 3.0), yaw_deg: Optional[float] = None,
                         shift=None, dtype: str = "f32") -> TemporalInputs:
    """An arbitrary-size seeded temporal case; ``yaw_deg`` / ``shift`` fix the motion."""
    cur = random_case(5000 + seed, B, N, C, H, W, X, Y, Z, rng6=rng6, dtype=dtype, with_grad=False)
    prev = np.random.default_rng([5000 + seed, 1]).standard_normal((B, Cp, X, Y), dtype=np.float32)
    g = np.random.default_rng([5000 + seed, 2]).standard_normal((B, C + Cp, X, Y), dtype=np.float32)
    return TemporalInputs(cur, prev, make_ego_motion(5000 + seed, B, yaw_deg, shift), g)
