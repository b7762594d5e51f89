"""Host logic of bench.py's profile summaries (no GPU): the trace table's
timed-steps column and the traffic record's source hash."""
import csv
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _write_csv(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=list(rows[0].keys()))
        w.writeheader()
        w.writerows(rows)


def test_trace_summary_timed_steps_mean(tmp_path, monkeypatch):
    """The added column is the mean of each kernel's last N dispatches, N from
    the command's --steps; kernels with fewer dispatches get an empty cell."""
    trace = tmp_path / "trace"
    trace.mkdir()
    durs = [300, 250, 200, 100, 110, 120]   # warm-up first, then 3 timed steps
    _write_csv(trace / "run_kernel_stats.csv", [
        {"Name": "k_a", "Calls": len(durs), "AverageNs": sum(durs) / len(durs), "MinNs": min(durs),
         "MaxNs": max(durs), "Percentage": 90.0},
        {"Name": "k_b", "Calls": 1, "AverageNs": 5, "MinNs": 5, "MaxNs": 5, "Percentage": 10.0}])
    rows, t = [], 0
    for d in durs:
        rows.append({"Kernel_Name": "k_a", "Start_Timestamp": t, "End_Timestamp": t + d})
        t += 1000
    rows.append({"Kernel_Name": "k_b", "Start_Timestamp": t, "End_Timestamp": t + 5})
    _write_csv(trace / "run_kernel_trace.csv", rows)
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    bench.trace_summary(str(trace), "title", "python3 bench.py --steps 3 --warmup 3", "out")
    text = (tmp_path / "out.md").read_text()
    line_a = next(l for l in text.splitlines() if l.startswith("| `k_a`"))
    line_b = next(l for l in text.splitlines() if l.startswith("| `k_b`"))
    assert "average ns, last 3 dispatches" in text
    assert line_a.rstrip().endswith("| 110 |")      # (100 + 110 + 120) / 3
    assert line_b.rstrip().endswith("% | |")        # one dispatch: no timed-steps mean


def test_trace_summary_without_steps_has_no_column(tmp_path, monkeypatch):
    trace = tmp_path / "trace"
    trace.mkdir()
    _write_csv(trace / "run_kernel_stats.csv", [
        {"Name": "k", "Calls": 2, "AverageNs": 10, "MinNs": 9, "MaxNs": 11, "Percentage": 100.0}])
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    bench.trace_summary(str(trace), "title", "python3 bench.py", "out")
    assert "last" not in (tmp_path / "out.md").read_text()


def test_source_hash_tracks_content(tmp_path):
    a, b = tmp_path / "a.hip", tmp_path / "b.hip"
    a.write_text("x")
    b.write_text("y")
    h1 = bench.source_hash([str(a), str(b)])
    assert h1 == bench.source_hash([str(a), str(b)])
    b.write_text("y // changed")
    assert bench.source_hash([str(a), str(b)]) != h1
