"""bench.py's profile summaries, on synthetic rocprofv3 result databases.

The summaries turn rocprofv3's `kernels` and `pmc_events` views into the
tables under profiles/ and into profiles/traffic.json, which bench.py then
reports as `roofline.traffic`.  These tests build small databases with the
same columns, with known durations and counter values, and check the
arithmetic: per-(kernel, grid) grouping, the copy calibration, and which
dispatches make up one prefill call.  No GPU is needed.
"""
import json
import os
import sqlite3
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

NS = "void jscan_detail::"
PASS1 = NS + "k_scan<unsigned short, false, false, false, false, 1>(unsigned short const*, ...)"
PASS2 = NS + "k_scan<unsigned short, false, false, false, false, 2>(unsigned short const*, ...)"
COMBINE = NS + "k_combine<unsigned short>(float const*, ...)"
STEP = NS + "k_step<unsigned short, false, false, false, false>(float*, ...)"
COPY = "__amd_rocclr_copyBuffer"


def make_db(path, dispatches, counter=None):
    """dispatches: (name, grid, duration_ns, counter_kib_per_instance); two
    counter instances per dispatch, as a counter summed over several blocks."""
    con = sqlite3.connect(path)
    con.execute("create table kernels (dispatch_id, name, grid_x, grid_y, grid_z, start, duration)")
    con.execute("create table pmc_events (dispatch_id, counter_name, counter_value)")
    for i, (name, grid, dur, kib) in enumerate(dispatches):
        con.execute("insert into kernels values (?,?,?,?,?,?,?)", (i, name, *grid, i * 1000, dur))
        if counter is not None:
            for _ in range(2):
                con.execute("insert into pmc_events values (?,?,?)", (i, counter, kib / 2))
    con.commit()
    con.close()


def test_trace_summary_groups_by_kernel_and_grid(tmp_path):
    db = str(tmp_path / "trace.db")
    make_db(db, [(PASS1, (8192, 32, 1), 1_500_000, 0), (PASS1, (8192, 32, 1), 1_600_000, 0),
                 (PASS1, (8192, 16, 2), 900_000, 0), (STEP, (8388608, 1, 1), 54_000, 0)])
    out = str(tmp_path / "trace.md")
    stats = bench.summarize_trace(db, out, "cmd")
    assert stats[(bench.PASS1, "8192x32x1")] == [1500.0, 1600.0]      # microseconds
    assert stats[(bench.PASS1, "8192x16x2")] == [900.0]
    text = open(out).read()
    assert "| k_scan<unsigned short, false, false, false, false, 1> | 8192x32x1 | 2 | 1550.0 |" in text
    assert "cmd" in text


def test_traffic_summary_calibrates_and_assembles_one_call(tmp_path):
    gib_kib = (1 << 30) / 1024
    # FETCH_SIZE reads half the bytes of the 1 GiB copy, WRITE_SIZE all of them
    fetch = [(COPY, (131072, 1, 1), 0, gib_kib / 2), (COPY, (65536, 1, 1), 0, 10.0),
             (PASS1, (8192, 32, 1), 0, 1000.0), (PASS1, (8192, 32, 1), 0, 1200.0), (PASS1, (8192, 32, 1), 0, 1100.0),
             (PASS2, (8192, 31, 1), 0, 100.0), (PASS2, (8192, 15, 2), 0, 5000.0),
             (COMBINE, (131072, 1, 1), 0, 10.0), (STEP, (8388608, 1, 1), 0, 300.0),
             (STEP, (4194304, 1, 1), 0, 150.0)]
    write = [(COPY, (131072, 1, 1), 0, gib_kib), (COPY, (65536, 1, 1), 0, 10.0),
             (PASS1, (8192, 32, 1), 0, 400.0), (PASS1, (8192, 32, 1), 0, 400.0), (PASS1, (8192, 32, 1), 0, 400.0),
             (PASS2, (8192, 31, 1), 0, 50.0), (PASS2, (8192, 15, 2), 0, 2000.0),
             (COMBINE, (131072, 1, 1), 0, 5.0), (STEP, (8388608, 1, 1), 0, 200.0),
             (STEP, (4194304, 1, 1), 0, 100.0)]
    for sub, rows, counter in (("fetch", fetch, "FETCH_SIZE"), ("write", write, "WRITE_SIZE")):
        os.makedirs(tmp_path / "pmc" / sub)
        make_db(str(tmp_path / "pmc" / sub / "run_results.db"), rows, counter)
    out_json = str(tmp_path / "traffic.json")
    bench.summarize_traffic(str(tmp_path / "pmc"), str(tmp_path / "traffic.md"), out_json, "cmd")
    data = json.load(open(out_json))
    assert data["fetch_scale"] == pytest.approx(2.0) and data["write_scale"] == pytest.approx(1.0)
    kib = 1024.0
    p1 = (1100.0 * 2 + 400.0) * kib                # medians, scaled
    p2 = (100.0 * 2 + 50.0) * kib                  # pass 2's own grid, not the 8192x15x2 one
    cmb = (10.0 * 2 + 5.0) * kib
    assert data["prefill_64k"]["hbm_bytes_per_launch"] == pytest.approx(p1)
    assert data["prefill_64k"]["whole_call_bytes"] == pytest.approx(p1 + p2 + cmb)
    assert data["prefill_64k"]["alg_bytes"] == bench.alg_bytes_prefill(1, 65536, 8192)
    assert data["decode_256"]["hbm_bytes_per_launch"] == pytest.approx((300.0 * 2 + 200.0) * kib)
    assert data["prefill_64k"]["source_sha"] == bench.source_digest()


def test_algorithmic_bytes():
    """The survey's accounting: 8 bytes per channel-token plus 64 per token of
    B and C rows, A and D, and the final state; 136 per channel-token for the
    decode step plus the rows and parameters."""
    assert bench.alg_bytes_prefill(1, 65536, 8192) == 4300242944
    assert bench.alg_bytes_prefill(1, 65536, 8192) / (65536 * 8192) == pytest.approx(8.01, abs=0.01)
    assert bench.alg_bytes_step(256, 8192) == 285786112
    assert bench.alg_bytes_step(256, 8192) / (256 * 8192) == pytest.approx(136.3, abs=0.05)


def test_more_than_one_gpu_is_refused():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_code_digest_ignores_comments_only():
    """The counters in profiles/traffic.json stay valid across comment edits of
    the kernel sources and lapse on any change to the code itself."""
    code = 'h[n] = fmaf(e, h[n], dx * B[n]);  // state\n/* a note */ const char* s = "// kept";\n'
    assert bench._code_only(code) == bench._code_only(code.replace("// state", "// the state update"))
    assert bench._code_only(code) == bench._code_only(code.replace("/* a note */", "/* another\n note */"))
    assert bench._code_only(code) != bench._code_only(code.replace("dx * B[n]", "dx * C[n]"))
    assert bench._code_only(code) != bench._code_only(code.replace('"// kept"', '"// changed"'))
