"""bench.py's contract on the host: one GPU only (a clear exit for more),
the committed HBM-traffic summary belongs to the score kernel as it is,
and the CPU baseline leg reports the oracle's rate with its core count."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_summary_matches_the_score_source():
    """profiles/ holds FETCH/WRITE counters taken on this fm_score.hip: the
    bench reads its bytes per launch (about 1.014x the algorithmic 136 B per
    chunk at B=30, N=262144)."""
    t = bench.read_traffic(30 * 262144)
    assert t is not None, "counter summary missing or taken on another version of fm_score.hip"
    algorithmic = 30 * 262144 * bench.SCORE_BYTES_PER_CHUNK
    assert 0.99 * algorithmic < t < 1.10 * algorithmic


def test_cpu_baseline_reports_the_oracle():
    b = bench.cpu_baseline(0.0)  # one row, the least the leg times
    assert b["kind"] == "oracle" and b["unit"] == "chunks/s"
    assert b["value"] > 0 and b["cores"] >= 1
    assert b["sample"].startswith("1 of 30 rows")
