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


def test_traffic_summary_tied_to_the_score_source(tmp_path):
    """The bench reads HBM bytes per launch from a counter summary only when
    the summary's digest is that of the score kernel's sources as they are;
    a stale summary gives null.  When the committed summary is current, its
    bytes are about the algorithmic 136 B per chunk at B=30, N=262144."""
    algorithmic = 30 * 262144 * bench.SCORE_BYTES_PER_CHUNK
    good = tmp_path / "good.txt"
    good.write_text(f"# x\nscore_source_sha256: {bench.source_digest()}\nhbm_bytes_per_launch: 1084266125\n")
    assert bench.read_traffic(30 * 262144, str(good)) == 1084266125.0
    stale = tmp_path / "stale.txt"
    stale.write_text("score_source_sha256: " + "0" * 64 + "\nhbm_bytes_per_launch: 1084266125\n")
    assert bench.read_traffic(30 * 262144, str(stale)) is None
    assert bench.read_traffic(30 * 262144, str(tmp_path / "missing.txt")) is None
    t = bench.read_traffic(30 * 262144)
    if t is not None:
        assert 0.99 * algorithmic < t < 1.10 * algorithmic


def test_source_digest_covers_the_shared_score_headers():
    names = [os.path.basename(p) for p in bench.SCORE_SRCS]
    assert {"fm_score.hip", "fm_score_common.h", "fm_internal.h", "fm_index.h"} <= set(names)


def test_cpu_baseline_reports_the_oracle():
    """One row, the least the leg times, plus the oracle's resident delta and
    subset top-K on small host inputs standing in for the legs' copies."""
    rng = np.random.default_rng(0)
    legs = {"resident_delta": (rng.random((2, 600)) < 0.1, rng.random((2, 600)) < 0.1),
            "subset_topk": (rng.random((2, 600)).astype(np.float32),
                            rng.permutation(600)[:300].astype(np.int32)[None].repeat(2, 0))}
    b = bench.cpu_baseline(0.0, legs)
    assert b["kind"] == "oracle" and b["unit"] == "chunks/s"
    assert b["parity"] is None and b["configs"] == {}
    assert b["value"] > 0 and b["cores"] >= 1
    assert b["sample"].startswith("1 of 30 rows")
    assert b["next_rows"]["resident_delta_us"] > 0 and b["next_rows"]["subset_topk_us"] > 0
    assert bench.cpu_baseline(0.0, {})["next_rows"] == {}


def test_cpu_baseline_times_and_checks_the_other_workloads():
    """Per workload, the leg times the oracle on whole rows of the inputs the
    GPU leg ran on and compares the GPU's outputs with the oracle's: here
    the oracle's own outputs stand in for the GPU's, so every difference is
    zero; a flipped mask entry far from the cut-off counts as outside the
    band."""
    import oracle
    import synth
    wl = synth.WORKLOADS[1]
    weights = synth.make_weights()
    inp = {"hidden": synth.make_hidden(wl), "positions": synth.make_positions(wl),
           "valid_n": synth.make_valid_n(wl), "comp_k": synth.make_comp_k(wl)}
    ref = oracle.run_row(weights, inp["hidden"][0], int(inp["positions"][0]), inp["comp_k"][0],
                         oracle.OracleConfig(), mode="max", top_k=512)
    inp["scores"] = ref["scores"][None].astype(np.float32)
    inp["mask"] = ref["mask"][None].copy()
    b = bench.cpu_baseline(0.0, {}, {1: inp}, config_budget_s=0.0)
    c = b["configs"][wl.name]
    assert c["rows"] == 1 and c["valid_chunks"] == 4096 and c["value"] > 0
    assert c["parity"]["rows"] == 1 and c["parity"]["max_abs_score_err"] < 1e-7
    assert c["parity"]["mask_diff_outside_band"] == 0
    low = int(np.argmin(ref["scores"]))
    inp["mask"][0, low] ^= 1
    c = bench.cpu_baseline(0.0, {}, {1: inp}, config_budget_s=0.0)["configs"][wl.name]
    assert c["parity"]["mask_diff_outside_band"] == 1


def test_only_the_cpu_baseline_leg_reaches_the_oracle():
    """The GPU legs of bench.py never import or call the oracle (the parity
    helpers take the oracle's outputs from the CPU-baseline leg)."""
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


def test_source_digest_ignores_comments_not_code():
    """A comment edit leaves the compiled kernel, and so the counters, as they
    were; a code edit voids them."""
    base = "int a = 1;  // one\n/* block\n comment */\nint b = 2;\n"
    assert bench._code_only(base) == bench._code_only("int a = 1;  // uno\n\nint b = 2;  /* two */\n")
    assert bench._code_only(base) != bench._code_only("int a = 1;\nint b = 3;\n")
