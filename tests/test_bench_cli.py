"""bench.py on the host: one GPU only (it says so for more), and its kernel
source hash ignores comments and whitespace but not code."""

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
