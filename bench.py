#!/usr/bin/env python3
"""Benchmark of the fused Sampling-VT hot path on one MI355X.

One step = one pass of the whole path over one batch: fbev_forward (voxel
centres, projection, validity, bilinear gather, valid-camera mean, height
sum) followed by fbev_backward (zero-fill + atomic scatter of dL/dF) on the
nuScenes-shaped workload: B=1, N=6 cameras, C=64, 16x44 fp32 features,
200x200 BEV cells over +-50 m, Z=8 height bins over [-5, 3) m, seeded
synthetic rig and N(0,1) features and upstream gradient.  Inputs are resident
in HBM before timing starts.

Prints one JSON line.  ``value`` is BEV output elements per second of whole
steps; per-pass figures (output elems/s, bilinear samples/s, algorithmic
HBM GB/s) follow in ``forward`` / ``backward``; ``roofline`` covers the
dominant kernel; ``cpu_baseline`` times the fp64 CPU oracle on the same
workload (a reported baseline, not a target).

``--workload`` selects another seeded workload: tiny, batched, large, fwdbwd
(single-level), pyramid (the multi-level path, fbev_forward_levels +
fbev_backward_levels on 32x88 / 16x44 / 8x22 levels of a 6-camera rig), or
lss / lss_batched (Lift-Splat, the push view transform: fbev_lss_forward +
fbev_lss_backward with 41 depth bins and 64 context channels per pixel), or
deform / deform_bev (Deformable Aggregation: fbev_deform_forward +
fbev_deform_backward for 900 sparse queries x 13 keypoints, or one query per
cell of a 200 x 200 grid x 8 keypoints), or cameras (the gradients of the
Sampling-VT output with respect to K, R and t, fbev_backward_cameras, on the
nuScenes-shaped workload), or temporal (fbev_forward_temporal +
fbev_backward_temporal: the nuScenes-shaped transform stacked with a 64-channel
previous BEV map resampled under a seeded ego motion).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "BEV output elems/s + bilinear samples/s; achieved HBM GB/s vs MI355X peak"
HBM_PEAK_GBPS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "camera_bev_view_amd", "csrc", "sampling_vt.hip")
LSS_SRC = os.path.join(ROOT, "camera_bev_view_amd", "csrc", "lift_splat.hip")
DEFORM_SRC = os.path.join(ROOT, "camera_bev_view_amd", "csrc", "deform_agg.hip")
CAMERA_SRC = os.path.join(ROOT, "camera_bev_view_amd", "csrc", "camera_grad.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
# The host dispatch chooses lane layouts, tile shapes and instantiations: counters taken before a change
# to these files no longer describe the launched kernels, so every traffic record must carry their hashes.
DISPATCH_SRCS = ("camera_bev_view_amd/csrc/kernels.h", "camera_bev_view_amd/csrc/flashbev_api.cpp")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), for the CPU-baseline record."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def kernel_source_hash(path: str = KERNEL_SRC) -> str:
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def measured_traffic(kernel, workload: str, field: str = "bytes_per_launch"):
    """A per-launch figure from committed rocprofv3 PMC counters (``field``: HBM bytes, or
    ``valu_insts`` for SQ_INSTS_VALU), or None when they were taken on a different kernel
    source or workload (or never).  Each workload's record names the source file(s) its
    counters were taken on.  ``kernel`` may be a list: the sum over one pass of those kernels."""
    if isinstance(kernel, (list, tuple)):
        parts = [measured_traffic(k, workload, field) for k in kernel]
        return None if any(v is None for v in parts) else sum(parts)
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    w = rec.get("workloads", {}).get(workload, {})
    sources = w.get("sources") or {w.get("source", os.path.relpath(KERNEL_SRC, ROOT)):
                                   w.get("source_sha256", rec.get("source_sha256"))}
    if any(d not in sources for d in DISPATCH_SRCS):
        return None
    try:
        if any(sha != kernel_source_hash(os.path.join(ROOT, src)) for src, sha in sources.items()):
            return None
    except OSError:
        return None
    k = w.get("kernels", {}).get(kernel)
    return k.get(field) if k else None


# Vector-ALU issue peak without packed math: 256 CUs x 4 SIMDs x 16 lanes, one lane-operation per cycle
# each at 2.4 GHz (a wave64 instruction occupies its SIMD for 4 cycles).
VALU_PEAK_LANE_OPS = 256 * 4 * 16 * 2.4e9


def counter_fracs(kernels, ms, workload):
    """``valu_frac`` (SQ_INSTS_VALU x 64 lanes / time / VALU_PEAK_LANE_OPS) and ``hbm_frac_counters``
    (FETCH_SIZE + WRITE_SIZE bytes / time / 8 TB/s) of a pass of ``kernels`` taking ``ms``, from the
    committed counters (None when missing or stale)."""
    s_ = ms * 1e-3
    valu = measured_traffic(kernels, workload, "valu_insts")
    traffic = measured_traffic(kernels, workload)
    return {"valu_frac": None if valu is None else valu * 64 / s_ / VALU_PEAK_LANE_OPS,
            "hbm_frac_counters": None if traffic is None else traffic / s_ / 1e9 / HBM_PEAK_GBPS}


def pass_roofline(kernels, rate, nbytes, workload):
    """The ``roofline`` object of one timed pass: algorithmic bytes over the pass's HIP-event time.
    ``kernels`` lists the pass's launches in order (their rocprofv3 durations add up to the pass);
    ``traffic`` sums their counter bytes (None when the counters are missing or stale)."""
    achieved = rate["hbm_gbps_algorithmic"]
    d = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
         "frac": achieved / HBM_PEAK_GBPS,
         "traffic": measured_traffic(kernels, workload),
         "kernel": " + ".join(kernels), "launch_ms": rate["ms"], "algorithmic_bytes": nbytes}
    d.update(counter_fracs(kernels, rate["ms"], workload))
    return d


def time_floor(args, dev, shape):
    """The compulsory part of a forward pass: a torch ``fill_`` of an fp32 tensor of the output's shape
    on the same stream (one launch and a write-only pass over the output), timed like the passes."""
    import numpy as np
    import torch
    buf = torch.empty(shape, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        buf.fill_(1.0)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k, (a, b) in enumerate(ev):
        a.record(stream)
        buf.fill_(float(k))
        b.record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    log(f"[bench] floor: fill of {tuple(shape)} fp32 {ms * 1e3:.2f} us")
    return ms


def time_passes(args, dev, passes, label):
    """W untimed warm-up steps, then K timed steps of ``passes`` (callables, run in order on the current
    stream) bracketed by synchronizations, with nothing else in the stream between them; then, untimed for
    the step rate, up to 100 more steps with HIP events around every pass (an event between two kernels adds
    a few microseconds of its own, so the step rate is taken without them).  Returns (ms per step over the
    timed region, [mean ms of each pass]).  The host stays at most ~64 steps ahead of the GPU (it waits on
    an event recorded 64 steps earlier), so a long run never fills the stream's queue, past which every
    launch would wait for a free slot.  With --cold a 1 GiB buffer is overwritten before every timed step
    (more than the L2s and the 256 MB Infinity Cache hold), so each step starts with its inputs in HBM only;
    the step time is then the sum of each step's own passes, HIP events around every pass of every step."""
    import numpy as np
    import torch
    log(f"[bench] warmup {args.warmup} steps on {label}")
    for _ in range(args.warmup):
        for f in passes:
            f()
    torch.cuda.synchronize()
    calibration_copy(args, dev)
    stream = torch.cuda.current_stream(dev)
    n = len(passes)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    ahead = 64
    marks = {}

    def run(steps, ev=None, sweep=None):
        for k in range(steps):
            if k >= ahead and (k - ahead) in marks:
                marks.pop(k - ahead).synchronize()
            if sweep is not None:
                sweep.fill_(float(k))
            for i, f in enumerate(passes):
                if ev is not None:
                    ev[k][i].record(stream)
                f()
            if ev is not None:
                ev[k][n].record(stream)
            if k % 16 == 0:
                marks[k] = torch.cuda.Event()
                marks[k].record(stream)
        marks.clear()

    if args.cold:
        sweep = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(args.steps)]
        log(f"[bench] timing {args.steps} steps (cold: cache sweep before each)")
        torch.cuda.synchronize()
        run(args.steps, ev, sweep)
        torch.cuda.synchronize()
        ms_step = float(np.mean([e[0].elapsed_time(e[n]) for e in ev]))
    else:
        log(f"[bench] timing {args.steps} steps")
        torch.cuda.synchronize()
        t_start.record(stream)
        run(args.steps)
        t_end.record(stream)
        torch.cuda.synchronize()
        ms_step = t_start.elapsed_time(t_end) / args.steps
        n_ev = min(args.steps, 100)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(n_ev)]
        run(n_ev, ev)
        torch.cuda.synchronize()
    pass_ms = [float(np.mean([e[i].elapsed_time(e[i + 1]) for e in ev])) for i in range(n)]
    log(f"[bench] done: {ms_step * 1e3:.2f} us/step (passes " + ", ".join(f"{m * 1e3:.2f}" for m in pass_ms) + " us)")
    return ms_step, pass_ms


def pass_rates(ms, nbytes, **counts):
    """Per-pass figures: ``counts`` (items per pass) become items/s; algorithmic HBM GB/s and fraction."""
    s_ = ms * 1e-3
    d = {"ms": ms}
    for k, v in counts.items():
        d[k] = v / s_
    d.update({"algorithmic_bytes": nbytes, "hbm_gbps_algorithmic": nbytes / s_ / 1e9,
              "hbm_frac_algorithmic": nbytes / s_ / 1e9 / HBM_PEAK_GBPS})
    return d


def bench_line(args, value, ms_step, dtype, data, config):
    """The JSON line's fixed fields, in order."""
    if args.cold:
        config = dict(config, cache="cold: 1 GiB overwritten before every timed step")
    return {"metric": METRIC, "value": value, "unit": "BEV output elems/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": dtype, "data": data, "config": config}


def calibration_copy(args, dev):
    """A plain copy of --calib-copy-mib MiB, three times, for scaling the HBM byte counters."""
    if not args.calib_copy_mib:
        return
    import torch
    n = args.calib_copy_mib * (1 << 20) // 4
    src = torch.randn(n, device=dev)
    dst = torch.empty_like(src)
    # an elementwise kernel (a plain device-to-device copy_ may go to a DMA engine,
    # which the shader counters do not see): reads and writes n floats once
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    log(f"[bench] calibration copy of {args.calib_copy_mib} MiB done (x3)")


def cpu_baseline_levels(inp, rows):
    """Time the multi-level fp64 oracle (forward + backward) on the first ``rows`` X-rows."""
    import oracle.multilevel as ml
    sel = list(range(rows))
    t0 = time.perf_counter()
    c0 = time.process_time()
    ml.oracle_forward_levels(inp.levels, inp.K, inp.R, inp.t, inp.rng6, inp.X, inp.Y, inp.Z, rows=sel)
    ml.oracle_backward_levels(inp.grad_out, inp.K, inp.R, inp.t, inp.rng6, inp.X, inp.Y, inp.Z, inp.shapes, rows=sel)
    wall = time.perf_counter() - t0
    cpu = time.process_time() - c0
    B, C = inp.levels[0].shape[0], inp.levels[0].shape[2]
    return {
        "value": B * C * rows * inp.Y / wall,
        "unit": "BEV output elems/s",
        "cores": max(1, round(cpu / wall)),
        "kind": "oracle",
        "sample": f"fp64 numpy multi-level oracle, forward + backward over X-rows 0..{rows - 1} of {inp.X} "
                  f"({B * C * rows * inp.Y} outputs), wall {wall:.2f} s, process CPU {cpu:.2f} s, "
                  f"{len(os.sched_getaffinity(0))} cores available, {cpu_model()}",
    }


def cpu_baseline(inp, rows):
    """Time the fp64 oracle (forward + backward) on the first ``rows`` X-rows."""
    import numpy as np
    import oracle
    H, W = inp.F.shape[-2:]
    sel = list(range(rows))
    t0 = time.perf_counter()
    c0 = time.process_time()
    oracle.oracle_forward(inp.F, inp.K, inp.R, inp.t, inp.rng6, inp.X, inp.Y, inp.Z, rows=sel)
    oracle.oracle_backward(inp.grad_out, inp.K, inp.R, inp.t, inp.rng6, inp.X, inp.Y, inp.Z, H, W, rows=sel)
    wall = time.perf_counter() - t0
    cpu = time.process_time() - c0
    B, C = inp.F.shape[0], inp.F.shape[2]
    return {
        "value": B * C * rows * inp.Y / wall,
        "unit": "BEV output elems/s",
        "cores": max(1, round(cpu / wall)),
        "kind": "oracle",
        "sample": f"fp64 numpy oracle, forward + backward over X-rows 0..{rows - 1} of {inp.X} "
                  f"({B * C * rows * inp.Y} outputs), wall {wall:.2f} s, process CPU {cpu:.2f} s, "
                  f"{len(os.sched_getaffinity(0))} cores available, {cpu_model()}",
    }


def cpu_baseline_lss(inp, min_seconds=10.0):
    """Time the fp64 Lift-Splat oracle (forward + backward) on whole steps, repeated for ``min_seconds``."""
    import oracle.lift_splat as ls
    reps = 0
    t0 = time.perf_counter()
    c0 = time.process_time()
    while True:
        ls.lss_forward(inp.depth, inp.context, inp.K, inp.R, inp.t, inp.rng6, inp.X, inp.Y, inp.d_min, inp.d_step)
        ls.lss_backward(inp.grad_out, inp.depth, inp.context, inp.K, inp.R, inp.t, inp.rng6, inp.X, inp.Y,
                        inp.d_min, inp.d_step)
        reps += 1
        wall = time.perf_counter() - t0
        if wall >= min_seconds:
            break
    cpu = time.process_time() - c0
    B, C = inp.context.shape[0], inp.context.shape[2]
    return {
        "value": reps * B * C * inp.X * inp.Y / wall,
        "unit": "BEV output elems/s",
        "cores": max(1, round(cpu / wall)),
        "kind": "oracle",
        "sample": f"fp64 numpy Lift-Splat oracle, {reps} whole forward + backward steps of the workload, "
                  f"wall {wall:.2f} s, process CPU {cpu:.2f} s, {len(os.sched_getaffinity(0))} cores available, "
                  f"{cpu_model()}",
    }


def main_lss(args):
    """Lift-Splat: one step = fbev_lss_forward + fbev_lss_backward on one batch."""
    import numpy as np
    import torch
    from camera_bev_view_amd import ops
    from camera_bev_view_amd import workloads as wl

    dev = torch.device("cuda:0")
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    inp = wl.make_lss_inputs(args.workload, with_grad=True)
    B, N, D, H, W = inp.depth.shape
    C = inp.context.shape[2]
    X, Y = inp.X, inp.Y
    dep = to_dev(inp.depth.transpose(0, 1, 3, 4, 2))
    ctx = to_dev(inp.context.transpose(0, 1, 3, 4, 2))
    K, R, t = (to_dev(a) for a in (inp.K, inp.R, inp.t))
    g = to_dev(inp.grad_out)
    out = torch.empty((B, C, X, Y), dtype=torch.float32, device=dev)
    gd = torch.empty_like(dep)
    gc = torch.empty_like(ctx)
    geo = (inp.rng6, X, Y, inp.d_min, inp.d_step)
    fwd_call = lambda: ops.lss_forward(dep, ctx, K, R, t, *geo, out=out)
    bwd_call = lambda: ops.lss_backward(g, dep, ctx, K, R, t, *geo, grad_depth=gd, grad_context=gc)

    ms_step, (fwd_ms, bwd_ms) = time_passes(args, dev, [fwd_call, bwd_call], args.workload)
    out_elems = B * C * X * Y
    pix = B * N * H * W
    points = pix * D
    cam_bytes = B * N * 21 * 4
    fwd_bytes = pix * (D + C) * 4 + out_elems * 4 + cam_bytes            # alpha and c once, output once
    bwd_bytes = out_elems * 4 + 2 * pix * (D + C) * 4 + cam_bytes         # grad_out, alpha and c once; both grads once
    fwd = pass_rates(fwd_ms, fwd_bytes, out_elems_per_s=out_elems, lifted_points_per_s=points)
    bwd = pass_rates(bwd_ms, bwd_bytes, out_elems_per_s=out_elems, lifted_points_per_s=points)
    # the timed passes: the forward kernel alone; the backward's zero-fill (both gradients) and its kernel
    dom_k, dom, dom_bytes = (["lift_splat_fwd"], fwd, fwd_bytes) if fwd_ms >= bwd_ms else \
        (["lss_fill_zero", "lift_splat_bwd"], bwd, bwd_bytes)
    line = bench_line(args, out_elems / (ms_step * 1e-3), ms_step, "f32",
                      "synthetic: seeded 6-camera ring rig, flat-Dirichlet depth distributions, N(0,1) context and "
                      "upstream gradient",
                      {"workload": f"{args.workload}: Lift-Splat B={B} N={N} HxW={H}x{W} D={D} bins "
                                   f"{inp.d_min}+k*{inp.d_step} m, C={C} -> X*Y={X}x{Y} pillars, "
                                   f"one step = forward + backward",
                       "B": B, "N": N, "C": C, "H": H, "W": W, "D": D, "X": X, "Y": Y})
    line.update({"lifted_points_per_s": points * 2 / (ms_step * 1e-3), "forward": fwd, "backward": bwd,
                 "roofline": pass_roofline(dom_k, dom, dom_bytes, args.workload)})
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline")
        line["cpu_baseline"] = cpu_baseline_lss(inp)
    print(json.dumps(line), flush=True)


def cpu_baseline_deform(inp, max_queries, min_seconds=10.0):
    """Time the fp64 Deformable Aggregation oracle (forward + backward) on the first ``max_queries``
    queries, repeated until ``min_seconds`` have passed."""
    import oracle.deform_agg as da
    Qs = min(max_queries, inp.anchors.shape[1])
    sl = (slice(None), slice(0, Qs))
    args = (inp.F, inp.K, inp.R, inp.t, inp.anchors[sl], inp.offsets[sl], inp.weights[sl])
    reps = 0
    in_view = 0
    t0 = time.perf_counter()
    c0 = time.process_time()
    while True:
        ref = da.deform_forward(*args)
        da.deform_backward(inp.grad_out[sl], *args)
        in_view = int(ref["valid"].sum())
        reps += 1
        wall = time.perf_counter() - t0
        if wall >= min_seconds:
            break
    cpu = time.process_time() - c0
    B, C = inp.F.shape[0], inp.F.shape[2]
    return {
        "value": reps * B * Qs * C / wall,
        "unit": "BEV output elems/s",
        "cores": max(1, round(cpu / wall)),
        "kind": "oracle",
        "sample": f"fp64 numpy Deformable Aggregation oracle, {reps} forward + backward passes over queries "
                  f"0..{Qs - 1} of {inp.anchors.shape[1]} (output elements = queries x channels), wall {wall:.2f} s, "
                  f"process CPU {cpu:.2f} s, {len(os.sched_getaffinity(0))} cores available, {cpu_model()}",
        "in_view_samples_in_sample": in_view,
    }


def main_deform(args):
    """Deformable Aggregation: one step = fbev_deform_forward + fbev_deform_backward on one batch."""
    import numpy as np
    import torch
    from camera_bev_view_amd import ops
    from camera_bev_view_amd import workloads as wl

    dev = torch.device("cuda:0")
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    inp = wl.make_deform_inputs(args.workload, with_grad=True)
    B, N, C, H, W = inp.F.shape
    Q, Kp = inp.offsets.shape[1:3]
    F = to_dev(inp.F.transpose(0, 1, 3, 4, 2))
    K, R, t = (to_dev(a) for a in (inp.K, inp.R, inp.t))
    A, D, Wt = to_dev(inp.anchors), to_dev(inp.offsets), to_dev(inp.weights)
    g = to_dev(inp.grad_out)
    out = torch.empty((B, Q, C), dtype=torch.float32, device=dev)
    fwd_call = lambda: ops.deform_forward(F, K, R, t, A, D, Wt, out=out)
    bwd_call = lambda: ops.deform_backward(g, F, K, R, t, A, D, Wt)

    ms_step, (fwd_ms, bwd_ms) = time_passes(args, dev, [fwd_call, bwd_call], args.workload)
    out_elems = B * Q * C
    feat_bytes = B * N * H * W * C * 4
    q_bytes = B * Q * (3 + 3 * Kp + N * Kp) * 4
    fwd_bytes = feat_bytes + q_bytes + out_elems * 4 + B * N * 21 * 4
    bwd_bytes = out_elems * 4 + 2 * feat_bytes + 2 * q_bytes + B * N * 21 * 4
    fwd = pass_rates(fwd_ms, fwd_bytes, out_elems_per_s=out_elems)
    bwd = pass_rates(bwd_ms, bwd_bytes, out_elems_per_s=out_elems)
    dom_k, dom, dom_bytes = (["deform_fwd"], fwd, fwd_bytes) if fwd_ms >= bwd_ms else \
        (["deform_fill_zero", "deform_bwd", "deform_scan_apply", "deform_scatter", "deform_gather4"], bwd, bwd_bytes)
    line = bench_line(args, out_elems / (ms_step * 1e-3), ms_step, "f32",
                      "synthetic: seeded 6-camera ring rig, N(0,1) features and upstream gradient, seeded anchors and "
                      "offsets, flat-Dirichlet weights",
                      {"workload": f"{args.workload}: Deformable Aggregation B={B} N={N} C={C} HxW={H}x{W} Q={Q} "
                                   f"queries x Kp={Kp} keypoints (outputs = query features), one step = forward + "
                                   f"backward", "B": B, "N": N, "C": C, "H": H, "W": W, "Q": Q, "Kp": Kp})
    line.update({"forward": fwd, "backward": bwd, "roofline": pass_roofline(dom_k, dom, dom_bytes, args.workload)})
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline")
        line["cpu_baseline"] = cpu_baseline_deform(inp, 4000)
    print(json.dumps(line), flush=True)


def cpu_baseline_cameras(inp, min_seconds=10.0):
    """Time the fp64 camera-gradient oracle over the whole grid, repeated until ``min_seconds`` have passed."""
    import oracle.camera_grad as cg
    reps = 0
    t0 = time.perf_counter()
    c0 = time.process_time()
    while True:
        cg.oracle_camera_backward(inp.grad_out, inp.F, inp.K, inp.R, inp.t, inp.rng6, inp.X, inp.Y, inp.Z)
        reps += 1
        wall = time.perf_counter() - t0
        if wall >= min_seconds:
            break
    cpu = time.process_time() - c0
    B, C = inp.F.shape[0], inp.F.shape[2]
    return {
        "value": reps * B * C * inp.X * inp.Y / wall,
        "unit": "BEV output elems/s",
        "cores": max(1, round(cpu / wall)),
        "kind": "oracle",
        "sample": f"fp64 numpy camera-gradient oracle, {reps} whole passes over the {inp.X}x{inp.Y}x{inp.Z} grid, "
                  f"wall {wall:.2f} s, process CPU {cpu:.2f} s, {len(os.sched_getaffinity(0))} cores available, "
                  f"{cpu_model()}",
    }


def main_cameras(args):
    """Camera gradients: one step = fbev_backward_cameras (gather pass + fixed-order finish) on one batch."""
    import numpy as np
    import torch
    from camera_bev_view_amd import ops
    from camera_bev_view_amd import workloads as wl

    dev = torch.device("cuda:0")
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    inp = wl.make_inputs("nuscenes", with_grad=True)
    B, N, C, H, W = inp.F.shape
    X, Y, Z = inp.X, inp.Y, inp.Z
    F = to_dev(inp.F.transpose(0, 1, 3, 4, 2))
    K, R, t = (to_dev(a) for a in (inp.K, inp.R, inp.t))
    g = to_dev(inp.grad_out)
    ws = torch.empty((1 << 24,), dtype=torch.uint8, device=dev)
    call = lambda: ops.camera_backward(g, F, K, R, t, inp.rng6, X, Y, Z, workspace=ws)

    ms_step, (pass_ms,) = time_passes(args, dev, [call], "cameras")
    out_elems = B * C * X * Y
    nbytes = B * N * H * W * C * 4 + out_elems * 4 + B * N * 21 * 4 * 2   # features, grad_out, cameras in, gradients out
    rate = pass_rates(pass_ms, nbytes)
    line = bench_line(args, out_elems / (ms_step * 1e-3), ms_step, "f32",
                      "synthetic: seeded 6-camera ring rig, N(0,1) features and upstream gradient",
                      {"workload": f"cameras: dL/dK, dL/dR, dL/dt of the Sampling-VT, B={B} N={N} C={C} "
                                   f"HxW={H}x{W} grid {X}x{Y}x{Z} (outputs = the BEV elements whose gradient is "
                                   f"pulled back)", "B": B, "N": N, "C": C, "H": H, "W": W, "X": X, "Y": Y, "Z": Z})
    line.update({"pass": {"ms": pass_ms, "algorithmic_bytes": nbytes, "hbm_gbps_algorithmic": rate["hbm_gbps_algorithmic"]},
                 "roofline": pass_roofline(["camera_grad_main", "camera_grad_finish"], rate, nbytes, "cameras")})
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline")
        line["cpu_baseline"] = cpu_baseline_cameras(inp)
    print(json.dumps(line), flush=True)


def cpu_baseline_temporal(ti, min_seconds=10.0):
    """Time the fp64 temporal oracle (forward + backward) over the whole grid until ``min_seconds`` have passed."""
    import oracle.temporal as tp
    cur = ti.cur
    B, N, C, H, W = cur.F.shape
    reps = 0
    t0 = time.perf_counter()
    c0 = time.process_time()
    while True:
        tp.temporal_forward(cur.F, cur.K, cur.R, cur.t, cur.rng6, cur.X, cur.Y, cur.Z, ti.prev, ti.ego)
        tp.temporal_backward(ti.grad_out, cur.K, cur.R, cur.t, cur.rng6, cur.X, cur.Y, cur.Z, H, W, C, ti.ego)
        reps += 1
        wall = time.perf_counter() - t0
        if wall >= min_seconds:
            break
    cpu = time.process_time() - c0
    Cp = ti.prev.shape[1]
    return {
        "value": reps * B * (C + Cp) * cur.X * cur.Y / wall,
        "unit": "BEV output elems/s",
        "cores": max(1, round(cpu / wall)),
        "kind": "oracle",
        "sample": f"fp64 numpy temporal oracle (Sampling-VT + resampled previous map), {reps} forward + backward "
                  f"passes over the whole {cur.X}x{cur.Y} grid, wall {wall:.2f} s, process CPU {cpu:.2f} s, "
                  f"{len(os.sched_getaffinity(0))} cores available, {cpu_model()}",
    }


def main_temporal(args):
    """Temporal fused transform: one step = fbev_forward_temporal + fbev_backward_temporal on one batch."""
    import numpy as np
    import torch
    from camera_bev_view_amd import ops
    from camera_bev_view_amd import workloads as wl

    dev = torch.device("cuda:0")
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    ti = wl.make_temporal_inputs(args.workload)
    cur = ti.cur
    B, N, C, H, W = cur.F.shape
    X, Y, Z = cur.X, cur.Y, cur.Z
    Cp = ti.prev.shape[1]
    F = to_dev(cur.F.transpose(0, 1, 3, 4, 2))
    K, R, t = (to_dev(a) for a in (cur.K, cur.R, cur.t))
    prev, ego, g = to_dev(ti.prev), to_dev(ti.ego), to_dev(ti.grad_out)
    out = torch.empty((B, C + Cp, X, Y), dtype=torch.float32, device=dev)
    fwd_call = lambda: ops.forward_temporal(F, K, R, t, cur.rng6, X, Y, Z, prev, ego, out=out)
    bwd_call = lambda: ops.backward_temporal(g, (B, N, H, W, C), K, R, t, cur.rng6, X, Y, Z, Cp, ego)

    ms_step, (fwd_ms, bwd_ms) = time_passes(args, dev, [fwd_call, bwd_call], args.workload)
    out_elems = B * (C + Cp) * X * Y
    cams = B * N * 21 * 4 + B * 6 * 4
    feat_bytes = B * N * H * W * C * 4
    fwd_bytes = feat_bytes + B * Cp * X * Y * 4 + out_elems * 4 + cams       # features, previous map, output
    bwd_bytes = out_elems * 4 + feat_bytes + B * Cp * X * Y * 4 + cams       # upstream gradient, dL/dF, dL/dprev
    fwd = pass_rates(fwd_ms, fwd_bytes, out_elems_per_s=out_elems)
    bwd = pass_rates(bwd_ms, bwd_bytes, out_elems_per_s=out_elems)
    # the backward: zero-fill, the bin-run Sampling-VT backward and the resampling adjoint (maps of at most
    # 256 x 256 pixels), else zero-fill and the fused hash-table kernel
    bwd_k = ["fill_zero_f32", "sampling_vt_runs_bwd", "bev_align_bwd"] if max(H, W) <= 256 else \
        ["fill_zero_f32", "temporal_bwd"]
    # the forward: one launch of the bin-run kernel's tiles and the resampling units where the channels take the
    # 16-byte, 16-lane layout (256 bytes per pixel), else the hash-era forward fused with the resampling
    fwd_k = ["temporal_runs_fwd"] if C * 4 == 256 else ["temporal_fwd"]
    dom_k, dom, dom_bytes = (fwd_k, fwd, fwd_bytes) if fwd_ms >= bwd_ms else (bwd_k, bwd, bwd_bytes)
    line = bench_line(args, out_elems / (ms_step * 1e-3), ms_step, "f32",
                      "synthetic: seeded 6-camera ring rig, N(0,1) features, previous map and upstream gradient, "
                      "seeded planar ego motion",
                      {"workload": f"{args.workload}: Sampling-VT B={B} N={N} C={C} HxW={H}x{W} grid {X}x{Y}x{Z} "
                                   f"stacked with a Cp={Cp} previous BEV map resampled under the ego motion, one step "
                                   f"= forward + backward", "B": B, "N": N, "C": C, "Cp": Cp, "H": H, "W": W, "X": X,
                       "Y": Y, "Z": Z})
    line.update({"forward": fwd, "backward": bwd, "roofline": pass_roofline(dom_k, dom, dom_bytes, args.workload)})
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline")
        line["cpu_baseline"] = cpu_baseline_temporal(ti)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="nuscenes")
    ap.add_argument("--dtype", default=None)
    ap.add_argument("--cpu-rows", type=int, default=None, help="X-rows of the CPU-oracle sample (default: all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold", action="store_true", help="overwrite 1 GiB before every timed step (cold caches)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path would shard by batch sample or BEV rows with no exchange in the forward; "
              "only the one-GPU measurement is implemented)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from camera_bev_view_amd import ops
    from camera_bev_view_amd import workloads as wl

    if args.workload in wl.LSS_WORKLOADS:
        return main_lss(args)
    if args.workload in wl.DEFORM_WORKLOADS:
        return main_deform(args)
    if args.workload == "cameras":
        return main_cameras(args)
    if args.workload in wl.TEMPORAL_WORKLOADS:
        return main_temporal(args)
    dev = torch.device("cuda:0")
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    if args.workload in wl.PYRAMIDS:
        # multi-level (feature-pyramid) path: packed level features [B,N,P,C]
        inp = wl.make_level_inputs(args.workload, dtype=args.dtype, with_grad=True)
        B, N, C = inp.levels[0].shape[:3]
        H, W = inp.shapes[0]
        nlev = len(inp.shapes)
        lv = [torch.from_numpy(np.ascontiguousarray(F.transpose(0, 1, 3, 4, 2))) for F in inp.levels]
        if inp.dtype == "bf16":
            lv = [x.to(torch.bfloat16) for x in lv]
        Fdev = ops.pack_levels([x.to(dev) for x in lv])
        P = Fdev.shape[2]
        desc = f"levels {'/'.join(f'{h}x{w}' for h, w in inp.shapes)}"
        fwd_call = lambda **kw: ops.forward_levels(Fdev, inp.shapes, K, R, t, inp.rng6, X, Y, Z, **kw)
        bwd_call = lambda: ops.backward_levels(g, B, N, C, inp.shapes, K, R, t, inp.rng6, X, Y, Z)
        baseline = cpu_baseline_levels
    else:
        inp = wl.make_inputs(args.workload, dtype=args.dtype, with_grad=True)
        B, N, C, H, W = inp.F.shape
        nlev, P = 1, H * W
        Fdev = torch.from_numpy(np.ascontiguousarray(inp.F.transpose(0, 1, 3, 4, 2)))
        if inp.dtype == "bf16":
            Fdev = Fdev.to(torch.bfloat16)
        Fdev = Fdev.to(dev)
        desc = f"HxW={H}x{W}"
        fwd_call = lambda **kw: ops.forward(Fdev, K, R, t, inp.rng6, X, Y, Z, **kw)
        bwd_call = lambda: ops.backward(g, (B, N, H, W, C), K, R, t, inp.rng6, X, Y, Z)
        baseline = cpu_baseline
    X, Y, Z = inp.X, inp.Y, inp.Z
    K, R, t = (to_dev(a) for a in (inp.K, inp.R, inp.t))
    g = to_dev(inp.grad_out)
    out = torch.empty((B, C, X, Y), dtype=torch.float32, device=dev)
    es = Fdev.element_size()
    # the key of this run's counter record: the workload, plus the dtype when it is not the workload's first
    first = wl.WORKLOADS[args.workload].dtypes[0] if args.workload in wl.WORKLOADS else "f32"
    key = args.workload if inp.dtype == first else f"{args.workload}_{inp.dtype}"

    # valid (cell, z, camera) samples, for the samples/s figures (outside the timed region)
    _, cnt = fwd_call(with_counts=True)
    torch.cuda.synchronize()
    valid_tuples = int(cnt.to(torch.int64).sum().item())
    del cnt

    ms_step, (fwd_ms, bwd_ms) = time_passes(args, dev, [lambda: fwd_call(out=out), bwd_call], args.workload)
    out_elems = B * C * X * Y
    cam_bytes = B * N * 21 * 4
    feat_bytes = B * N * P * C * es
    fwd_bytes = feat_bytes + out_elems * 4 + cam_bytes            # features once, output once
    bwd_bytes = out_elems * 4 + B * N * P * C * 4 + cam_bytes      # grad_out once, dL/dF once
    samples = valid_tuples * C * nlev                              # one bilinear sample per level
    logical = B * N * C * X * Y * Z * nlev
    fwd = pass_rates(fwd_ms, fwd_bytes, out_elems_per_s=out_elems, bilinear_samples_per_s=samples,
                     logical_samples_per_s=logical)
    bwd = pass_rates(bwd_ms, bwd_bytes, out_elems_per_s=out_elems, bilinear_samples_per_s=samples,
                     logical_samples_per_s=logical)
    # the timed passes: the forward kernel alone; the backward's zero-fill and its kernel (one launch, all
    # feature levels; the bin-run kernel for single-level maps of at most 256 x 256 pixels)
    fwd_k = ["sampling_vt_runs_fwd"]
    bwd_k = ["fill_zero_f32", "sampling_vt_runs_bwd" if nlev == 1 and max(H, W) <= 256 else "sampling_vt_bwd"]
    fwd.update(counter_fracs(fwd_k, fwd_ms, key))
    bwd.update(counter_fracs(bwd_k, bwd_ms, key))
    floor_ms = time_floor(args, dev, (B, C, X, Y))
    fwd["roofline"] = dict(pass_roofline(fwd_k, fwd, fwd_bytes, key), floor_ms=floor_ms,
                           floor_frac=floor_ms / fwd_ms)
    dom_k, dom, dom_bytes = (fwd_k, fwd, fwd_bytes) if fwd_ms >= bwd_ms else (bwd_k, bwd, bwd_bytes)
    line = bench_line(args, out_elems / (ms_step * 1e-3), ms_step,
                      "f32" if inp.dtype == "f32" else "bf16 in, f32 accumulate",
                      "synthetic: seeded 6-camera ring rig, N(0,1) features and upstream gradient",
                      {"workload": f"{args.workload}: B={B} N={N} C={C} {desc} {inp.dtype} -> "
                                   f"X*Y*Z={X}x{Y}x{Z}, one step = forward + backward",
                       "B": B, "N": N, "C": C, "H": H, "W": W, "levels": nlev, "X": X, "Y": Y, "Z": Z,
                       "valid_samples_per_pass": valid_tuples})
    line.update({"bilinear_samples_per_s": samples * 2 / (ms_step * 1e-3), "forward": fwd, "backward": bwd,
                 "roofline": dict(pass_roofline(dom_k, dom, dom_bytes, key), floor_ms=floor_ms)})
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline")
        line["cpu_baseline"] = baseline(inp, args.cpu_rows or X)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
