"""bench.py's contract on the host: one GPU only (a clear exit for more),
the committed HBM-traffic summary belongs to the score kernel as it is,
and the CPU baseline leg, the only one that touches the oracle, reports its
rate with its core count."""

import os
import subprocess
import sys

import numpy as np
import pytest

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
    """One row, the least the leg times, plus the oracle's resident delta and
    subset top-K on small host inputs standing in for the legs' copies."""
    rng = np.random.default_rng(0)
    legs = {"resident_delta": (rng.random((2, 600)) < 0.1, rng.random((2, 600)) < 0.1),
            "subset_topk": (rng.random((2, 600)).astype(np.float32),
                            rng.permutation(600)[:300].astype(np.int32)[None].repeat(2, 0))}
    b = bench.cpu_baseline(0.0, legs)
    assert b["kind"] == "oracle" and b["unit"] == "chunks/s"
    assert b["value"] > 0 and b["cores"] >= 1
    assert b["sample"].startswith("1 of 30 rows")
    assert b["next_rows"]["resident_delta_us"] > 0 and b["next_rows"]["subset_topk_us"] > 0
    assert bench.cpu_baseline(0.0, {})["next_rows"] == {}


def test_only_the_cpu_baseline_leg_reaches_the_oracle():
    """The GPU legs of bench.py never import or call the oracle."""
    import ast
    import inspect
    tree = ast.parse(inspect.getsource(bench))
    for fn in tree.body:
        if isinstance(fn, ast.FunctionDef) and fn.name != "cpu_baseline":
            names = {n.id for n in ast.walk(fn) if isinstance(n, ast.Name)}
            mods = {a.name for n in ast.walk(fn) if isinstance(n, (ast.Import, ast.ImportFrom))
                    for a in n.names} | {n.module for n in ast.walk(fn) if isinstance(n, ast.ImportFrom)}
            assert "oracle" not in names and "oracle" not in mods, fn.name


@pytest.mark.gpu
def test_timing_event_brackets_the_same_work_as_torch_events():
    """bench.TimingEvent (no system-scope fence) times 20 fills of 256 MB
    within a few percent of torch's default events around the same work."""
    import torch
    x = torch.empty(1 << 26, device="cuda")
    s = torch.cuda.current_stream()
    for _ in range(3):
        x.fill_(1.0)
    torch.cuda.synchronize()
    a, b = bench.TimingEvent(), bench.TimingEvent()
    ta, tb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ta.record(s)
    a.record(s)
    for _ in range(20):
        x.fill_(2.0)
    b.record(s)
    tb.record(s)
    torch.cuda.synchronize()
    t_hip, t_torch = a.elapsed_time(b), ta.elapsed_time(tb)
    assert 0.8 * t_torch < t_hip <= 1.05 * t_torch + 0.01, (t_hip, t_torch)
    assert float(x[-1]) == 2.0
