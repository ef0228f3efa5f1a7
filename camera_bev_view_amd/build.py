"""Build libflashbev.so in-tree with hipcc for gfx950.

``python -m camera_bev_view_amd.build`` (or ``__graft_entry__.build()``)
compiles the C-ABI host layer and the HIP kernels into
``camera_bev_view_amd/libflashbev.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libflashbev.so")
SOURCES = [os.path.join(CSRC, "flashbev_api.cpp"), os.path.join(CSRC, "sampling_vt.hip"),
           os.path.join(CSRC, "lift_splat.hip"), os.path.join(CSRC, "deform_agg.hip"),
           os.path.join(CSRC, "camera_grad.hip"), os.path.join(CSRC, "temporal.hip"),
           os.path.join(CSRC, "sampling_vt_runs.hip")]
ARCH = "gfx950"

# Packed-fp32 VALU forms are switched off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-munsafe-fp-atomics"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libflashbev)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}: {' '.join(cmd[-3:])}")


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every source into libflashbev.so (always recompiles, one hipcc per source in parallel, then
    one link); returns its path."""
    from concurrent.futures import ThreadPoolExecutor
    obj_dir = os.path.join(ROOT, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    common = [hipcc(), "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-I", os.path.join(ROOT, "include"),
              *DEVICE_FLAGS, *extra_flags]
    objs = [os.path.join(obj_dir, os.path.basename(src) + ".o") for src in SOURCES]
    jobs = max(1, min(len(SOURCES), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(jobs) as pool:
        for f in [pool.submit(_run, common + ["-c", src, "-o", obj], verbose) for src, obj in zip(SOURCES, objs)]:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
