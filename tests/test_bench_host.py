"""Host-side logic of bench.py (no GPU): the one-GPU contract, the rocprofv3
summary it prints, and the rule that recorded HBM traffic is reported only
while the kernel sources still match the counter run."""

import os
import sqlite3
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, cwd=ROOT, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""          # no JSON line for a configuration it does not measure


def test_rocprof_summary_columns(tmp_path):
    db = tmp_path / "trace" / "bench_results.db"
    db.parent.mkdir()
    con = sqlite3.connect(db)
    con.execute("create table kernels(name text, start integer, end integer)")
    # 5 slow warm-up dispatches (3 us) then 20 timed ones (2 us), plus another kernel
    for i in range(25):
        con.execute("insert into kernels values (?, ?, ?)",
                    ("kern_a", 10_000 * i, 10_000 * i + (3000 if i < 5 else 2000)))
    con.execute("insert into kernels values ('kern_b', 5, 1005)")
    con.commit()
    con.close()
    r = run_bench("--rocprof-summary", str(db))
    assert r.returncode == 0, r.stderr
    lines = r.stdout.splitlines()
    assert lines[0] == "## trace/bench_results.db"
    assert lines[1].split()[:6] == ["calls", "avg_us", "min_us", "max_us", "median_us", "last_us"]
    a = next(l for l in lines if l.rstrip().endswith("kern_a")).split()
    assert int(a[0]) == 25
    assert float(a[1]) == pytest.approx(2.2)   # mean over all 25
    assert float(a[2]) == 2.0 and float(a[3]) == 3.0 and float(a[4]) == 2.0
    assert float(a[5]) == 2.0                   # mean of the last 20 (the timed steps)
    assert lines.index(next(l for l in lines if l.rstrip().endswith("kern_a"))) < \
        lines.index(next(l for l in lines if l.rstrip().endswith("kern_b")))   # by total time


def test_strip_comments_keeps_code():
    src = "int a = 1; // note\n/* block\n comment */ int b = 2;\n\n   \nint c;  \n"
    assert bench.strip_comments(src) == "int a = 1;\n int b = 2;\nint c;"


def test_traffic_only_for_matching_sources(monkeypatch):
    # rows of the committed traffic table: kernel | source hash | ... | bytes
    rows = {}
    with open(bench.TRAFFIC_TABLE) as fh:
        for line in fh:
            cells = [c.strip() for c in line.strip().strip("|").split("|")]
            if len(cells) >= 5 and cells[0] in ("fwd", "dkdv", "dq", "preprocess"):
                rows[cells[0]] = (cells[1], int(cells[4]))
    assert set(rows) == {"fwd", "dkdv", "dq", "preprocess"}
    # reported while the sources hash to the recorded value ...
    for k, (h, nbytes) in rows.items():
        monkeypatch.setattr(bench, "source_hash", lambda kernel, h=h: h)
        assert bench.measured_traffic(k) == nbytes
    # ... and not once they have changed since the counter run
    monkeypatch.setattr(bench, "source_hash", lambda kernel: "000000000000")
    assert bench.measured_traffic("dkdv") is None


def test_metric_and_data_follow_the_workload():
    assert bench.metric_name("bf16", True, 0, 8192, 128) == \
        "fwd+bwd attention TFLOPS (bf16, causal, N=8192, d=128) + % of MFMA peak"
    assert bench.metric_name("bf16", False, 0, 2048, 64) == \
        "fwd+bwd attention TFLOPS (bf16, non-causal, N=2048, d=64) + % of MFMA peak"
    assert bench.metric_name("fp32", True, 256, 4096, 64) == \
        "fwd+bwd attention TFLOPS (fp32, causal, window 256, N=4096, d=64) + % of MFMA peak"
