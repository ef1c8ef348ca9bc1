"""Host-side logic of bench.py (no GPU): the one-GPU rule, the algorithmic work model,
the vector-issue view and the committed counter file's format."""
import math
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_work_per_plane():
    # two active planes, 100 supported entries and 3 written / 2 read columns in total
    info = {"n_active_bf": 2, "support_entries": 100, "columns_written": 3, "columns_read": 2}
    n = 64
    w = bench.algorithmic_work(n, info)
    fft = 5 * n * math.log2(n)
    assert w["pass1"]["bytes"] == pytest.approx(8 * 50 + 8 * n * 1.5)
    assert w["pass1"]["flops"] == pytest.approx(1.5 * fft + 45 * 50)
    assert w["pass2"]["bytes"] == pytest.approx(8 * n * 1.0 + 4 * n * n / 32)
    assert w["pass2"]["flops"] == pytest.approx((n // 2) * fft + 23 * n * n)


def test_issue_view_arithmetic(monkeypatch):
    # 6.144e11 wave instructions per second: 256 CUs x 4 SIMDs x 2.4 GHz / 4 cycles
    assert bench.PEAK_VALU_ISSUE == pytest.approx(6.144e11)
    monkeypatch.setattr(bench, "_counter_line", lambda k: ["pass1", "h", "1", "2", "6.144e8"])
    v = bench.issue_view("pass1", 2.0)
    assert v["issue_ms"] == pytest.approx(1.0)
    assert v["frac"] == pytest.approx(0.5)
    monkeypatch.setattr(bench, "_counter_line", lambda k: ["pass1", "h", "1", "2"])
    assert bench.issue_view("pass1", 2.0) is None
    assert bench.measured_traffic("pass1") == 3.0
    monkeypatch.setattr(bench, "_counter_line", lambda k: None)
    assert bench.measured_traffic("pass1") is None and bench.issue_view("pass1", 1.0) is None


def test_counter_file_format():
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    stages = set()
    with open(path) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            parts = line.split()
            assert len(parts) == 5, line
            assert len(parts[1]) == 16
            read_b, write_b, insts = (float(x) for x in parts[2:])
            assert read_b > 0 and write_b > 0 and insts > 0
            stages.add(parts[0])
    assert {"pass1", "pass2", "pass1@1024", "pass2@1024"} <= stages
