"""Turn rocprofv3 result databases into the committed performance record.

For one bench workload, given the databases (``run_results.db``) of a kernel-trace run and of three
``--pmc`` runs of the same bench command (FETCH_SIZE, WRITE_SIZE, SQ_INSTS_VALU), this

  * merges into ``profiles/traffic_counters.json`` the per-launch HBM bytes of every kernel (the
    median FETCH_SIZE / WRITE_SIZE over its dispatches, in KiB, scaled by what the same counters read
    for the bench's calibration copy of a known size) and its median SQ_INSTS_VALU, together with the
    sha256 of the sources the counters were taken on (``bench.py`` ignores a record whose sources
    changed since);
  * writes ``profiles/<prefix>_<key>.md`` (prefix ``sampling_vt`` by default): the kernel-trace table,
    the traffic table and the instruction counts, with the commands that produced them.

Usage (from the repository root, after the rocprofv3 runs):

    python -m camera_bev_view_amd.profile_record --key nuscenes --title "..." \\
        --trace T/run_results.db --fetch F/run_results.db --write W/run_results.db \\
        --valu V/run_results.db --calib-mib 256 --command "rocprofv3 ..." [--command ...]
"""
from __future__ import annotations

import argparse
import collections
import hashlib
import json
import os
import re
import sqlite3
import statistics
from typing import Dict, List

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RECORD = os.path.join(ROOT, "profiles", "traffic_counters.json")
# the files whose contents decide the launched kernels of the Sampling-VT passes (the default --sources)
SOURCES = ("camera_bev_view_amd/csrc/sampling_vt.hip", "camera_bev_view_amd/csrc/sampling_vt_runs.hip",
           "camera_bev_view_amd/csrc/wave_ops.h", "camera_bev_view_amd/csrc/bev_align.h",
           "camera_bev_view_amd/csrc/kernels.h", "camera_bev_view_amd/csrc/flashbev_api.cpp")


def short_name(name: str) -> str:
    """``void fbev::(anonymous namespace)::k<4, 16, false>(args)`` -> ``k``."""
    n = name.replace("(anonymous namespace)", "")
    n = re.sub(r"^void\s+", "", n)
    n = re.split(r"[<(]", n, maxsplit=1)[0]
    return n.split("::")[-1].strip() or name


def dispatches(db: str, counter: str):
    """(full kernel name, value) of every dispatch (the counter summed over its instances)."""
    con = sqlite3.connect(db)
    rows = con.execute("select kernel_name, dispatch_id, value from counters_collection where counter_name = ?",
                       (counter,)).fetchall()
    con.close()
    per = collections.defaultdict(float)
    names = {}
    for k, d, v in rows:
        per[d] += v
        names[d] = k
    return [(names[d], v) for d, v in per.items()]


def counters(db: str, counter: str) -> Dict[str, List[float]]:
    """Per kernel of this library (short name): the counter's value of every dispatch."""
    out = collections.defaultdict(list)
    for k, v in dispatches(db, counter):
        if "fbev::" in k:
            out[short_name(k)].append(v)
    return out


def trace(db: str) -> Dict[str, List[float]]:
    """Per kernel (short name): the durations (us) of its dispatches."""
    con = sqlite3.connect(db)
    rows = con.execute("select name, start, end from kernels").fetchall()
    con.close()
    out = collections.defaultdict(list)
    for k, s, e in rows:
        out[short_name(k)].append((e - s) / 1e3)
    return out


def calibration(fetch_db: str, write_db: str, calib_bytes: int):
    """The calibration copy of ``calib_bytes`` (read and written once) is the dispatch of a kernel outside this
    library with the most FETCH_SIZE of its run (a library kernel can fetch more than the copy on a large
    workload); in the other run, the dispatch of the same kernel with the most WRITE_SIZE.
    Returns (name, fetch KiB, write KiB, fetch factor, write factor)."""
    fk, f = max(((k, v) for k, v in dispatches(fetch_db, "FETCH_SIZE") if "fbev::" not in k), key=lambda kv: kv[1])
    w = max(v for k, v in dispatches(write_db, "WRITE_SIZE") if k == fk)
    return short_name(fk), f, w, calib_bytes / (f * 1024.0), calib_bytes / (w * 1024.0)


def sha(path: str) -> str:
    with open(os.path.join(ROOT, path), "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--key", required=True, help="record key: the bench workload, plus _<dtype> when not its first")
    ap.add_argument("--title", required=True, help="one line describing the workload")
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--valu", required=True)
    ap.add_argument("--calib-mib", type=int, default=256)
    ap.add_argument("--command", action="append", default=[], help="a command that produced the inputs")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    ap.add_argument("--prefix", default="sampling_vt", help="summary file name prefix (kernel family)")
    ap.add_argument("--sources", default=",".join(SOURCES),
                    help="comma-separated files (from the repository root) that decide the recorded kernels")
    ap.add_argument("--family", default="Sampling-VT", help="kernel family named in the summary's heading")
    ap.add_argument("--record", default=RECORD, help="the JSON record to merge into")
    a = ap.parse_args(argv)

    fetch, write = counters(a.fetch, "FETCH_SIZE"), counters(a.write, "WRITE_SIZE")
    valu, waves = counters(a.valu, "SQ_INSTS_VALU"), counters(a.valu, "SQ_WAVES")
    cal_k, cal_f, cal_w, ff, wf = calibration(a.fetch, a.write, a.calib_mib << 20)
    kernels = {}
    for k in sorted(set(fetch) & set(write)):
        fk, wk = statistics.median(fetch[k]), statistics.median(write[k])
        rec = {"fetch_kib_raw": round(fk, 2), "write_kib_raw": round(wk, 2),
               "fetch_bytes": int(round(fk * 1024 * ff)), "write_bytes": int(round(wk * 1024 * wf))}
        rec["bytes_per_launch"] = rec["fetch_bytes"] + rec["write_bytes"]
        if k in valu:
            rec["valu_insts"] = int(round(statistics.median(valu[k])))
        if k in waves:
            rec["waves"] = int(round(statistics.median(waves[k])))
        kernels[k] = rec
    try:
        with open(a.record) as fh:
            record = json.load(fh)
    except (OSError, ValueError):
        record = {}
    record["about"] = ("per kernel launch: HBM bytes from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (KiB per "
                       "dispatch, median over the dispatches of each kernel) scaled by what the same counters read "
                       "for the bench's elementwise calibration copy (--calib-copy-mib) in the same run, and the "
                       "median SQ_INSTS_VALU; written by camera_bev_view_amd/profile_record.py")
    record.setdefault("workloads", {})[a.key] = {
        "sources": {s: sha(s) for s in a.sources.split(",") if s},
        "commands": a.command,
        "calibration": {"copy_kernel": cal_k, "copy_bytes": a.calib_mib << 20, "fetch_kib_read": cal_f,
                        "write_kib_read": cal_w, "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)},
        "kernels": kernels,
    }
    with open(a.record, "w") as fh:
        json.dump(record, fh, indent=1)
        fh.write("\n")

    tr = trace(a.trace)
    total = sum(sum(v) for v in tr.values())
    lines = [f"# {a.family} kernels, {a.key}: rocprofv3 kernel trace and counters (MI355X)", "", a.title, "",
             "Commands (from the repository root; `<out>` is a scratch directory):", ""]
    lines += [f"    {c}" for c in a.command]
    lines += ["", "## Kernel trace", "", "| kernel | calls | average (us) | min (us) | max (us) | share |",
              "|---|---|---|---|---|---|"]
    for k, v in sorted(tr.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| {k} | {len(v)} | {statistics.mean(v):.2f} | {min(v):.2f} | {max(v):.2f} | "
                     f"{100 * sum(v) / total:.1f}% |")
    lines += ["", f"## HBM traffic and VALU instructions per launch (calibration: `{cal_k}` of "
                  f"{a.calib_mib} MiB read FETCH {cal_f:.0f} KiB, WRITE {cal_w:.0f} KiB; factors {ff:.4f} / {wf:.4f})",
              "", "| kernel | FETCH KiB | WRITE KiB | fetch bytes | write bytes | total bytes | SQ_INSTS_VALU | SQ_WAVES |",
              "|---|---|---|---|---|---|---|---|"]
    for k, r in kernels.items():
        lines.append(f"| {k} | {r['fetch_kib_raw']:.1f} | {r['write_kib_raw']:.1f} | {r['fetch_bytes']:,} | "
                     f"{r['write_bytes']:,} | {r['bytes_per_launch']:,} | {r.get('valu_insts', 0):,} | "
                     f"{r.get('waves', 0):,} |")
    lines.append("")
    path = os.path.join(a.out, f"{a.prefix}_{a.key}.md")
    with open(path, "w") as fh:
        fh.write("\n".join(lines))
    print(f"wrote {path} and {a.record}")


if __name__ == "__main__":
    main()
