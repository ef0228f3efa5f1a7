"""Host logic of bench.py (no GPU): the one-GPU guard, the JSON line's fixed fields, the cold-cache
marker, the roofline fraction and the staleness rule of the committed traffic counters."""
import argparse
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2 and r.stdout == ""
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("cold", [False, True])
def test_bench_line_fields(cold):
    args = argparse.Namespace(steps=7, warmup=3, cold=cold)
    line = bench.bench_line(args, 1.5e9, 0.25, "f32", "synthetic", {"workload": "w"})
    assert list(line)[:12] == ["metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                               "higher_is_better", "scaling", "vs_baseline", "dtype", "data"]
    assert line["n_gpus"] == 1 and line["steps"] == 7 and line["warmup"] == 3 and line["vs_baseline"] is None
    assert line["config"]["workload"] == "w"
    assert ("cache" in line["config"]) == cold
    json.dumps(line)


def test_pass_roofline_fraction():
    rate = {"hbm_gbps_algorithmic": 400.0, "ms": 0.02}
    r = bench.pass_roofline(["k1", "k2"], rate, 8_000_000, "no-such-workload")
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and r["unit"] == "GB/s"
    assert r["frac"] == pytest.approx(0.05) and r["kernel"] == "k1 + k2" and r["traffic"] is None


def test_traffic_counters_follow_their_sources(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_bytes(b"kernel source v1")
    rel = os.path.relpath(src, bench.ROOT)
    sha = hashlib.sha256(b"kernel source v1").hexdigest()
    disp = tmp_path / "dispatch.cpp"
    disp.write_bytes(b"dispatch v1")
    drel = os.path.relpath(disp, bench.ROOT)
    dsha = hashlib.sha256(b"dispatch v1").hexdigest()
    monkeypatch.setattr(bench, "DISPATCH_SRCS", (drel,))
    rec = {"workloads": {"w": {"sources": {rel: sha, drel: dsha},
                               "kernels": {"a": {"bytes_per_launch": 100}, "b": {"bytes_per_launch": 23}}},
                         "nodispatch": {"sources": {rel: sha}, "kernels": {"a": {"bytes_per_launch": 100}}}}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("a", "nodispatch") is None     # no hash of the dispatch code: stale
    assert bench.measured_traffic("a", "w") == 100
    assert bench.measured_traffic(["a", "b"], "w") == 123
    assert bench.measured_traffic(["a", "missing"], "w") is None
    assert bench.measured_traffic("a", "other") is None
    disp.write_bytes(b"dispatch v2")              # the dispatch changed since the counters were taken
    assert bench.measured_traffic("a", "w") is None
    disp.write_bytes(b"dispatch v1")
    assert bench.measured_traffic("a", "w") == 100
    src.write_bytes(b"kernel source v2")          # the kernel changed since the counters were taken
    assert bench.measured_traffic("a", "w") is None


def test_cpu_model_is_named():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()
