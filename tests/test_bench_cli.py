"""bench.py on the host: one GPU only (it says so for more), its kernel
source hash ignores comments and whitespace but not code, and the profile
summarizer picks, sums and averages rocprofv3 rows as its summaries state."""

import os
import subprocess
import sys

from conftest import REPO

sys.path.insert(0, REPO)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(REPO, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, cwd=REPO, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    src = tmp_path / "k.h"
    src.write_text("int f(int x) { return x + 1; }  // one\n/* block */\n")
    monkeypatch.setattr(bench, "REPO", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ["k.h"])
    h0 = bench.kernel_source_hash()
    src.write_text("int f(int x)  {\n  return x + 1;  // another comment\n}\n")
    assert bench.kernel_source_hash() == h0
    src.write_text("int f(int x) { return x + 2; }\n")
    assert bench.kernel_source_hash() != h0


def _write_csv(path, header, rows):
    """A CSV as rocprofv3 writes it (fields with commas quoted)."""
    import csv

    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_steady_dispatches_take_one_kernel_in_launch_order(tmp_path):
    """Trace summaries: the dispatches of the one kernel named by the prefix,
    sorted by start time, without the warm-up ones; a prefix that names two
    kernels is refused."""
    path = tmp_path / "run_kernel_trace.csv"
    a, b = "void retro::k<12, 2>(Args)", "void retro::other<12>(Args)"
    rows = [(a, 500, 530), (b, 100, 900), (a, 100, 110), (a, 300, 320), (a, 200, 215)]
    _write_csv(path, ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    name, durs = bench.steady_dispatches(str(path), "void retro::k<12,", 1)
    assert name == a and durs == [15, 20, 30]
    assert bench.steady_dispatches(str(path), "void retro::k<12,", 0)[1] == [10, 15, 20, 30]
    try:
        bench.steady_dispatches(str(path), "void retro::", 0)
    except RuntimeError as exc:
        assert "expected one kernel" in str(exc)
    else:
        raise AssertionError("two kernels under one prefix must be refused")


def test_counter_means_sum_each_dispatch_then_average(tmp_path):
    """Counter summaries: a counter's rows of one dispatch (one per XCD or
    instance) add up, the first dispatch (warm-up) is left out, and the rest
    are averaged."""
    path = tmp_path / "run_counter_collection.csv"
    k = "void retro::k<12, 2>(Args)"
    rows = [(1, k, "FETCH_SIZE", 100.0), (1, k, "FETCH_SIZE", 100.0),
            (2, k, "FETCH_SIZE", 300.0), (2, k, "FETCH_SIZE", 100.0),
            (3, k, "FETCH_SIZE", 200.0), (3, k, "FETCH_SIZE", 400.0),
            (4, "void retro::other<12>(Args)", "FETCH_SIZE", 9e9)]
    _write_csv(path, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], rows)
    assert bench._counter_means(str(path), "void retro::k<12,") == {"FETCH_SIZE": (500.0, 2)}
    assert bench._counter_means(str(path), "void retro::k<12,", drop=0) == {"FETCH_SIZE": (400.0, 3)}


def test_stats_row_gives_the_timed_steps_their_own_row():
    lines = bench._stats_row("k", [1000.0, 3000.0, 5000.0, 7000.0], steps=2)
    timed = next(l for l in lines if l.startswith("| timed steps"))
    rest = next(l for l in lines if l.startswith("| all after warm-up"))
    assert timed == "| timed steps | 2 | 2.00 | 3.00 | 1.00 | 3.00 |"
    assert rest == "| all after warm-up | 4 | 4.00 | 5.00 | 1.00 | 7.00 |"
    assert not any(l.startswith("| timed steps") for l in bench._stats_row("k", [1000.0]))


def test_recorded_traffic_is_used_only_for_the_same_kernel_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    h = bench.kernel_source_hash()
    (tmp_path / "t_traffic.md").write_text(f"hbm_bytes_per_launch: 5.676e+08\nsource_sha256: {h}\n")
    assert bench.read_traffic("t") == 5.676e8
    (tmp_path / "t_traffic.md").write_text("hbm_bytes_per_launch: 5.676e+08\nsource_sha256: 0123456789abcdef\n")
    assert bench.read_traffic("t") is None
    assert bench.read_traffic("missing") is None
