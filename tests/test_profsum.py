"""Host-side checks of the rocprofv3 summaries (profsum) and of how bench.py reads the
committed counter summary. Tiny synthetic databases with the tables profsum queries
stand in for rocprofv3 output; no GPU is needed."""
import json
import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from sparse_attention_decode_scores_amd import profsum  # noqa: E402

SCORE = "void dsa::k_score_row<2, 4, 2>(signed char const*, signed char const*)"
FOREIGN = "void at::native::vectorized_elementwise_kernel<4>()"
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(...)>()"


def trace_db(path, rows):
    con = sqlite3.connect(path)
    con.execute("CREATE TABLE kernels (name TEXT, grid_x INT, grid_y INT, grid_z INT, workgroup_x INT, "
                "workgroup_y INT, workgroup_z INT, start INT, end INT)")
    con.executemany("INSERT INTO kernels VALUES (?, ?, ?, ?, ?, ?, ?, ?, ?)", rows)
    con.commit()
    con.close()


def counter_db(path, rows):
    con = sqlite3.connect(path)
    con.execute("CREATE TABLE counters_collection (kernel_name TEXT, dispatch_id INT, counter_name TEXT, "
                "value REAL)")
    con.executemany("INSERT INTO counters_collection VALUES (?, ?, ?, ?)", rows)
    con.commit()
    con.close()


def test_kernel_stats_and_passes(tmp_path):
    # the score kernel: three 10 us calls, then two 20 us calls (times in ns), and one
    # foreign kernel in between
    rows, t = [], 0
    for i, d in enumerate((10000, 10000, 10000, 20000, 20000)):
        rows.append((SCORE, 235 * 512, 1, 1, 512, 1, 1, t, t + d))
        t += 50000
        if i == 1:
            rows.append((FOREIGN, 64, 1, 1, 64, 1, 1, t, t + 5000))
            t += 50000
    db = str(tmp_path / "run_results.db")
    trace_db(db, rows)
    by = {r["name"]: r for r in profsum.kernel_stats(db)}
    s = by[SCORE]
    assert s["calls"] == 5 and s["grid"] == 235 * 512 and s["block"] == 512
    assert abs(s["avg_us"] - 14.0) < 1e-9 and s["min_us"] == 10.0 and s["max_us"] == 20.0
    assert abs(by[SCORE]["pct"] + by[FOREIGN]["pct"] - 100.0) < 1e-9
    # calls are grouped in start order; only library kernels are listed
    passes = profsum.kernel_passes(db, [("first", 3), ("second", 2), ("none", 4)])
    assert [(p["name"], p["pass"], p["calls"], p["avg_us"]) for p in passes] == [
        (SCORE, "first", 3, 10.0), (SCORE, "second", 2, 20.0)]
    # a directory holding the database is accepted too
    assert profsum.kernel_stats(str(tmp_path))[0]["calls"] == 5


def test_counter_summary_scales_by_the_copy_kernel(tmp_path):
    # the copy reads 256 MiB and writes 256 MiB per dispatch; its counters read half
    # the bytes for FETCH_SIZE (scale 2) and all of them for WRITE_SIZE (scale 1)
    f, w, out = (str(tmp_path / n) for n in ("f.db", "w.db", "c.json"))
    counter_db(f, [(COPY, 1, "FETCH_SIZE", 131072.0), (COPY, 2, "FETCH_SIZE", 131072.0),
                   (SCORE, 3, "FETCH_SIZE", 60.0), (SCORE, 3, "FETCH_SIZE", 40.0),  # one dispatch, two rows
                   (SCORE, 4, "FETCH_SIZE", 300.0), (FOREIGN, 5, "FETCH_SIZE", 7.0)])
    counter_db(w, [(COPY, 1, "WRITE_SIZE", 262144.0), (SCORE, 3, "WRITE_SIZE", 10.0)])
    profsum.main(["counters", "--fetch-db", f, "--write-db", w, "--config", "ctx300k", "--command-fetch", "a",
                  "--command-write", "b", "--out", out])
    with open(out) as fh:
        d = json.load(fh)
    assert d["config"] == "ctx300k" and d["kernel_source_sha"] == profsum.library_source_sha()
    assert d["copy_calibration"]["fetch_scale"] == 2.0 and d["copy_calibration"]["write_scale"] == 1.0
    assert set(d["kernels"]) == {"k_score"}
    k = d["kernels"]["k_score"]
    assert k["fetch_dispatches"] == 2 and k["write_dispatches"] == 1
    assert k["hbm_read_bytes_per_launch"] == 200 * 1024 * 2  # mean of 100 and 300 KiB, doubled
    assert k["hbm_write_bytes_per_launch"] == 10 * 1024
    assert k["hbm_bytes_per_launch"] == 200 * 1024 * 2 + 10 * 1024


def test_bench_reads_traffic_only_for_matching_sources(tmp_path, monkeypatch):
    import bench
    p = tmp_path / "counters.json"
    summary = {"config": "ctx300k", "kernel_source_sha": profsum.library_source_sha(),
               "kernels": {"k_score": {"hbm_bytes_per_launch": 123}}}
    p.write_text(json.dumps(summary))
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(p))
    assert bench.measured_traffic("ctx300k") == {"k_score": 123}
    assert bench.measured_traffic("ctx16k") == {}  # another workload
    summary["kernel_source_sha"] = "0" * 16  # taken from other kernel sources
    p.write_text(json.dumps(summary))
    assert bench.measured_traffic("ctx300k") == {}
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("ctx300k") == {}
