"""Host logic of camera_bev_view_amd/profile_record.py (no GPU): the counter calibration takes the copy
kernel outside the library even when a library kernel fetched more, and the per-kernel traffic is scaled by
the copy's factors."""
import json
import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from camera_bev_view_amd import profile_record as pr  # noqa: E402

COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::CopyFunctor>(int)"
BWD = "void fbev::(anonymous namespace)::sampling_vt_runs_bwd<false>(fbev::BwdRunArgs)"
FWD = "void fbev::(anonymous namespace)::sampling_vt_runs_fwd<4, 16, false, false, false>(fbev::RunArgs)"


def make_db(path, counter, rows):
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (kernel_name text, dispatch_id integer, counter_name text, "
                "value real)")
    con.executemany("insert into counters_collection values (?, ?, ?, ?)",
                    [(k, d, counter, v) for k, d, v in rows])
    con.commit()
    con.close()


def test_calibration_skips_library_kernels_that_fetch_more(tmp_path):
    mib = 256
    kib = mib * 1024
    fetch = str(tmp_path / "fetch.db")
    write = str(tmp_path / "write.db")
    # the library's backward fetches more than the copy; two counter instances per dispatch are summed
    make_db(fetch, "FETCH_SIZE", [(COPY, 1, kib / 4), (COPY, 1, kib / 4), (BWD, 2, 3 * kib), (FWD, 3, 100.0)])
    make_db(write, "WRITE_SIZE", [(COPY, 1, kib), (BWD, 2, 5 * kib), (FWD, 3, 50.0)])
    name, f, w, ff, wf = pr.calibration(fetch, write, mib << 20)
    assert name == "vectorized_elementwise_kernel"
    assert f == kib / 2 and w == kib
    assert abs(ff - 2.0) < 1e-12 and abs(wf - 1.0) < 1e-12


def test_record_scales_each_kernel_by_the_copy_factors(tmp_path):
    mib = 256
    kib = mib * 1024
    dbs = {}
    for ctr, rows in (("FETCH_SIZE", [(COPY, 1, kib / 2), (BWD, 2, 1000.0), (BWD, 5, 1200.0), (BWD, 6, 1100.0)]),
                      ("WRITE_SIZE", [(COPY, 1, kib), (BWD, 2, 400.0), (BWD, 5, 400.0)])):
        dbs[ctr] = str(tmp_path / f"{ctr}.db")
        make_db(dbs[ctr], ctr, rows)
    valu = str(tmp_path / "valu.db")
    con = sqlite3.connect(valu)
    con.execute("create table counters_collection (kernel_name text, dispatch_id integer, counter_name text, "
                "value real)")
    con.executemany("insert into counters_collection values (?, ?, ?, ?)",
                    [(BWD, 2, "SQ_INSTS_VALU", 10.0), (BWD, 2, "SQ_WAVES", 5.0)])
    con.commit()
    con.close()
    trace = str(tmp_path / "trace.db")
    con = sqlite3.connect(trace)
    con.execute("create table kernels (name text, start integer, end integer)")
    con.executemany("insert into kernels values (?, ?, ?)", [(BWD, 0, 34000), (COPY, 0, 1000)])
    con.commit()
    con.close()
    record = str(tmp_path / "traffic.json")
    pr.main(["--key", "unit", "--title", "a test record", "--trace", trace, "--fetch", dbs["FETCH_SIZE"],
             "--write", dbs["WRITE_SIZE"], "--valu", valu, "--calib-mib", str(mib), "--out", str(tmp_path),
             "--record", record, "--sources", "camera_bev_view_amd/csrc/kernels.h"])
    rec = json.load(open(record))["workloads"]["unit"]["kernels"]["sampling_vt_runs_bwd"]
    # median FETCH 1100 KiB x 2.0, WRITE 400 KiB x 1.0
    assert rec["fetch_bytes"] == int(round(1100 * 1024 * 2.0))
    assert rec["write_bytes"] == 400 * 1024
    assert rec["bytes_per_launch"] == rec["fetch_bytes"] + rec["write_bytes"]
    assert rec["valu_insts"] == 10 and rec["waves"] == 5
    assert os.path.exists(tmp_path / "sampling_vt_unit.md")
