"""Host logic of bench.py (no GPU): the one-GPU refusal, the rocprofv3 summary and its
counter calibration, and the check that the committed counter summary belongs to the
current streaming-kernel sources (otherwise the bench reports its traffic as null)."""
import csv
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)


def test_summarize_rocprof_calibrates_and_sums_traffic(tmp_path, capsys):
    """A copy of 1 GiB that the counters see as half its bytes gives factor 2, applied to
    the streaming kernel's mean FETCH_SIZE and WRITE_SIZE (KiB per dispatch)."""
    calib = 1 << 30
    (tmp_path / "trace").mkdir()
    _write_csv(tmp_path / "trace" / "run_kernel_stats.csv",
               ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"],
               [["stream_dense<1, 1, 0, true>", 10, 8000, 7000, 9000]])
    ctr = ["Kernel_Name", "Counter_Name", "Dispatch_Id", "Counter_Value"]
    copy_kib = calib / 1024 / 2
    _write_csv(tmp_path / "fetch_counter_collection.csv", ctr, [
        ["at::native::copy_kernel", "FETCH_SIZE", 1, copy_kib],
        ["nvfp4::stream_dense<1, 1, 0, true>", "FETCH_SIZE", 2, 10000.0],
        ["nvfp4::stream_dense<1, 1, 0, true>", "FETCH_SIZE", 3, 12000.0],
    ])
    _write_csv(tmp_path / "write_counter_collection.csv", ctr, [
        ["at::native::copy_kernel", "WRITE_SIZE", 1, copy_kib],
        ["nvfp4::stream_dense<1, 1, 0, true>", "WRITE_SIZE", 2, 30.0],
        ["nvfp4::stream_dense<1, 1, 0, true>", "WRITE_SIZE", 3, 50.0],
    ])
    bench.summarize_rocprof(str(tmp_path), calib_bytes=calib)
    out = capsys.readouterr().out
    assert "calls     10 avg_us     8.000" in out
    assert "factor 2.0000" in out
    want = (11000.0 + 40.0) * 1024 * 2
    line = [ln for ln in out.splitlines() if ln.startswith("traffic_bytes_per_launch:")]
    assert line and int(line[0].split(":")[1]) == int(want)


def test_summarize_rocprof_dispatch_percentiles(tmp_path, capsys):
    """Median, p10 and p90 of the dispatch durations in a kernel trace, per kernel."""
    rows = [["k_a", 1000 * i, 1000 * i + 1000 * (i + 1)] for i in range(10)]  # 1..10 us
    rows += [["k_b", 0, 5000]] * 3
    _write_csv(tmp_path / "run_kernel_trace.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
               rows)
    bench.summarize_rocprof(str(tmp_path), calib_bytes=1 << 30)
    out = capsys.readouterr().out
    line_a = [ln for ln in out.splitlines() if ln.strip().startswith("k_a")][0].split()
    assert line_a[2] == "10" and float(line_a[4]) == 5.5
    assert abs(float(line_a[6]) - 1.9) < 1e-9 and abs(float(line_a[8]) - 9.1) < 1e-9
    line_b = [ln for ln in out.splitlines() if ln.strip().startswith("k_b")][0].split()
    assert line_b[2] == "3" and float(line_b[4]) == 5.0


def test_spread_percentiles():
    sp = bench.spread([1.0, 2.0, 3.0, 4.0, 5.0])
    assert sp == {"us_med": 3.0, "us_p10": 1.4, "us_p90": 4.6, "replays": 5}


def test_committed_counter_summary_matches_the_kernel_sources():
    """The FETCH/WRITE summary under profiles/ names the hash of the streaming kernel's
    sources it was taken on; it must be the current one, so that the bench's roofline
    carries measured traffic. Editing those sources means retaking the counters."""
    t = bench.measured_traffic()
    assert t is not None, "profiles/stream_dense_decode_sweep_pmc.txt predates the kernel sources"
    assert 28_000_000 < t < 40_000_000  # about the sweep's 28.7 MB of algorithmic bytes
