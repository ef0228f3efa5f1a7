"""Helpers shared by the GPU parity tests: device upload and the parity rules.

Parity rules (GPU vs the fp64 oracle):
  * valid-camera counts bit-exact, except (b, x, y, z) with a sample within
    1e-4 px of an image edge (a legitimate rounding flip of the in-view test);
  * forward outputs within |d| <= 1e-4 + 1e-5 |ref|, except cells having such
    a near-edge sample at some height;
  * backward within 1e-3 relative L2.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

ATOL = 1e-4
RTOL = 1e-5
BWD_REL_L2 = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(inp, device="cuda:0"):
    """Channels-last device features of the input's dtype plus fp32 K, R, t."""
    F = torch.from_numpy(np.ascontiguousarray(inp.F.transpose(0, 1, 3, 4, 2)))
    F = F.to(torch.bfloat16) if inp.dtype == "bf16" else F
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return F.contiguous().to(device), dev(inp.K), dev(inp.R), dev(inp.t)


def check_forward(out, counts, ref, rows=None, label="", exact_edges=False):
    """Apply the parity rules; ``rows`` selects the X-rows the oracle computed.
    ``exact_edges`` compares near-edge samples too (for cases built so that the
    projections land on an edge exactly, with no rounding to flip the test)."""
    out = out.float().cpu().numpy()
    if rows is not None:
        out = out[:, :, rows]
    ne = np.zeros_like(ref["near_edge"]) if exact_edges else ref["near_edge"]
    if counts is not None:
        cnt = counts.cpu().numpy()
        if rows is not None:
            cnt = cnt[:, rows]
        ok = ~ne
        mism = int(((cnt != ref["counts"]) & ok).sum())
        assert mism == 0, f"{label}: {mism} count mismatches"
    cell_ok = ~ne.any(axis=-1)
    diff = np.abs(out - ref["out"])
    tol = ATOL + RTOL * np.abs(ref["out"])
    bad = (diff > tol) & cell_ok[:, None]
    say(f"[parity] {label}: max|d|={diff[:, :][np.broadcast_to(cell_ok[:, None], diff.shape)].max(initial=0):.3e} "
        f"excluded cells={int((~cell_ok).sum())} excluded samples={int(ne.sum())}")
    assert not bad.any(), f"{label}: {int(bad.sum())} outputs outside tolerance, worst {diff[bad].max():.3e}"


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))
