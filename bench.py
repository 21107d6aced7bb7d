"""Benchmark of the Memory-Indexer scoring pass on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step = the whole pass over one batch: fm_prepare_query (query and weight
branches of the three layers) + fm_score (3-layer fused score, max
ensemble) + fm_select_topk (top-512 per row), on the B=30, N=262144
workload (a 1M-token context at 4x compression, concurrency 30), synthetic
seeded inputs already resident in HBM.  Prints one JSON line.

`roofline` describes the score kernel (the dominant one, MFMA-bound at
49152 flop per chunk); its duration comes from HIP events that libfm
records around the score kernel's own launch (fm_set_score_events), on
the stream the kernels run on; the whole fm_score call (query packing +
score kernel) is timed by events around it as well.  `traffic` is read from the
committed rocprofv3 counter summary when that summary was taken on the
current score-kernel source, else null.  `cpu_baseline` times the fp64
oracle on a bounded sample of the same workload on this host, and under
`next_rows` on the inputs the resident-delta and subset top-K legs ran on.
The next-row and variant legs run before the W warmup steps.  After the
warmup, untimed steps continue until at least --settle-seconds of
back-to-back load have run (the chip raises its clock over the first
fraction of a second of load after idle), then the K timed steps run.
`configs` times the other four seeded workloads (B=1 N=4096; B=8 N=65536
planted; B=32 N=131072 mean/threshold; B=60 N=131072 ragged YaRN top-1024)
the same way, each with its own oracle baseline; the headline `value` is
the B=30 N=262144 workload.  `mfma_ceiling` times dense f16 and bf16
GEMMs through torch.matmul (ROCm's BLAS) after a second of back-to-back
calls each: what a vendor-tuned MFMA kernel sustains on the same chip at
its power limit, set beside the score kernel's rate.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "chunks scored/s (3-layer fused score + top-K) and % of MFMA/HBM roofline"
WORKLOAD_ID = 5
TOP_K = 512
FLOP_PER_CHUNK = 3 * 64 * 128 * 2      # 49152 MFMA flop
EVENT_STRIDE = 5                       # per-phase events on every 5th timed step
SCORE_BYTES_PER_CHUNK = 132 + 4        # record read + ensemble score written
PEAK_F16_TFLOPS = 2500.0               # MI355X dense f16/bf16 MFMA
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5000.0               # MI355X dense fp8 MFMA
CSRC = os.path.join(ROOT, "sparse_attention_chunk_amd", "csrc")
# The score kernel's code and the constants it is built from: a change to
# any of them voids the committed counter summary.
SCORE_SRCS = [os.path.join(CSRC, f) for f in ("fm_score.hip", "fm_score_common.h", "fm_internal.h", "fm_index.h")]
QUERY_WEIGHT_BYTES = 3 * (1024 * 4096 + 1024 + 8192 * 1024 + 64 * 4096) * 4   # fp32 weights of the query branch
PMC_SUMMARY = os.path.join(ROOT, "profiles", "score_kernel_b30_n262144_pmc.txt")


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # The chip takes a few tens of steps after idle to reach its steady clock
    # under this load (five warmup steps alone would time that ramp); the
    # settle phase after the warmup covers it whatever W is.
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--settle-seconds", type=float, default=1.5,
                    help="untimed back-to-back steps after the warmup until this much load has run")
    ap.add_argument("--no-configs", action="store_true", help="time the headline workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing (profiling runs)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle time budget for the CPU baseline")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replayed step leg")
    ap.add_argument("--no-pipelined", action="store_true", help="skip the two-stream pipelined leg")
    ap.add_argument("--no-gemm-ceiling", action="store_true",
                    help="skip the dense f16 GEMM that gives the chip's sustained MFMA rate for comparison")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (for scaling FETCH_SIZE/WRITE_SIZE counters)")
    return ap.parse_args(argv)


def _code_only(text: str) -> str:
    """The source without its comments and blank lines (a comment edit does
    not change the compiled kernel, so it does not void the counters)."""
    import re

    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", line).rstrip() for line in text.splitlines())
    return "\n".join(line for line in lines if line)


def source_digest() -> str:
    """SHA-256 over the score kernel's sources (code only), in a fixed order."""
    h = hashlib.sha256()
    for path in SCORE_SRCS:
        with open(path, encoding="utf-8") as f:
            h.update(os.path.basename(path).encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()


def read_traffic(chunks_per_launch: int, summary: str = PMC_SUMMARY):
    """HBM bytes per score launch from the committed counter summary, or None
    if it is missing or was taken on another version of the score kernel."""
    if not os.path.exists(summary):
        return None
    vals = {}
    with open(summary) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("score_source_sha256") != source_digest():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class TimingEvent:
    """A HIP timing event created with hipEventDisableSystemFence.  A default
    event's record also writes back and invalidates the caches at system
    scope, which lengthens every interval it bounds by 1-2 us; this one only
    takes the timestamp.  Read it after a device synchronisation.  The HIP
    functions are looked up through libfm's handle, so they are those of the
    runtime libfm and torch share."""

    DISABLE_SYSTEM_FENCE = 0x20000000
    _hip = None

    def __init__(self):
        import ctypes

        if TimingEvent._hip is None:
            from sparse_attention_chunk_amd import _lib
            hip = _lib.LIB
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            TimingEvent._hip = hip
        self._ct = ctypes
        self.ev = ctypes.c_void_p()
        rc = TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream):
        rc = TimingEvent._hip.hipEventRecord(self.ev, self._ct.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end) -> float:
        """Milliseconds from this event to `end`, as torch.cuda.Event reports."""
        ms = self._ct.c_float()
        rc = TimingEvent._hip.hipEventElapsedTime(self._ct.byref(ms), self.ev, end.ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        try:
            if TimingEvent._hip is not None and self.ev:
                TimingEvent._hip.hipEventDestroy(self.ev)
        except Exception:  # interpreter shutdown
            pass


class ClockSampler:
    """Samples the GPU's firmware metrics (amdsmi gpu_metrics: GFX clocks,
    memory clock, socket power) from a background thread while running.
    The firmware reports clocks averaged over its own short window, which
    is closer to the shader clock kernels run at than the target clock the
    SMI's clock query shows.  Fails soft: summary() is None when amdsmi or
    the metrics table is unavailable."""

    KEYS = ("average_gfxclk_frequency", "current_gfxclk", "current_gfxclks", "current_uclk",
            "average_uclk_frequency", "average_socket_power", "current_socket_power")

    def __init__(self, period_s: float = 0.01):
        import threading
        self.period_s = period_s
        self.samples = []
        self._stop = threading.Event()
        self._thread = None
        self._handle = None
        self.error = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._amdsmi = amdsmi
            self._handle = amdsmi.amdsmi_get_processor_handles()[0]
            self._read()
        except Exception as e:  # no amdsmi, no metrics table, no permission
            self.error = f"{type(e).__name__}: {e}"
            self._handle = None

    def _read(self) -> dict:
        m = self._amdsmi.amdsmi_get_gpu_metrics_info(self._handle)
        out = {}
        for k in self.KEYS:
            v = m.get(k)
            if isinstance(v, (list, tuple)):
                v = [x for x in v if isinstance(x, (int, float)) and 0 < x < 65535]
                if v:
                    out[k] = sum(v) / len(v)
            elif isinstance(v, (int, float)) and 0 < v < 65535:
                out[k] = float(v)
        return out

    def _run(self):
        while not self._stop.is_set():
            try:
                self.samples.append(self._read())
            except Exception as e:  # pragma: no cover
                self.error = f"{type(e).__name__}: {e}"
                return
            self._stop.wait(self.period_s)

    def start(self):
        import threading
        self.samples = []
        self._stop.clear()
        if self._handle is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def stop(self):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()
            self._thread = None
        return self

    def summary(self):
        if self._handle is None or not self.samples:
            return None if self.error is None else {"error": self.error}
        out = {"samples": len(self.samples), "source": "amdsmi gpu_metrics"}
        for k in self.KEYS:
            vals = [smp[k] for smp in self.samples if k in smp]
            if vals:
                out[k] = {"mean": sum(vals) / len(vals), "min": min(vals), "max": max(vals)}
        return out


def settle(step, stream, min_s: float, block: int = 50):
    """Untimed back-to-back steps until at least min_s seconds of load have
    run, in blocks of `block` steps (one synchronisation per block).
    Returns the number of steps, the seconds and the per-step time of the
    first and last block (the clock ramp)."""
    import torch

    steps = 0
    per_block = []
    t0 = time.perf_counter()
    while True:
        t1 = time.perf_counter()
        for _ in range(block):
            step()
        torch.cuda.synchronize()
        per_block.append((time.perf_counter() - t1) / block)
        steps += block
        if time.perf_counter() - t0 >= min_s:
            break
    return {"steps": steps, "seconds": time.perf_counter() - t0, "first_block_us_per_step": per_block[0] * 1e6,
            "last_block_us_per_step": per_block[-1] * 1e6}


def _frac_at_clock(achieved_tflops: float, clocks: dict):
    """The score kernel's rate against the f16 MFMA peak scaled to the mean
    GFX clock the firmware reported during the settle phase (the published
    2.5 PF assumes 2.4 GHz), or None without clock samples."""
    try:
        mhz = float(clocks["current_gfxclk"]["mean"])
    except (KeyError, TypeError, ValueError):
        return None
    if not mhz > 0:
        return None
    peak = PEAK_F16_TFLOPS * mhz / 2400.0
    return {"gfxclk_mhz": mhz, "peak_tflops_at_clock": peak, "frac": achieved_tflops / peak,
            "note": "mean of the firmware's current_gfxclk samples over the settle phase"}


def graph_step_leg(body, outputs, steps: int, settle_s: float) -> dict:
    """The step captured once in a HIP graph (torch.cuda.CUDAGraph) and
    replayed: after settle_s seconds of replays, `steps` replays back to
    back, timed by host wall-clock between synchronisations and by two HIP
    events.  body(stream_handle) enqueues one step; `outputs` are the
    tensors it writes, whose eager values the last replay must equal bit
    for bit."""
    import torch

    torch.cuda.synchronize()
    eager = [t.clone() for t in outputs]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        body(side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        body(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    settled = settle(g.replay, stream, settle_s)
    ev = [TimingEvent() for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for _ in range(steps):
        g.replay()
    ev[1].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    ev_s = ev[0].elapsed_time(ev[1]) * 1e-3 / steps
    same = all(torch.equal(a, b) for a, b in zip(eager, outputs))
    del g
    return {"us_per_step": wall * 1e6, "us_per_step_events": ev_s * 1e6, "replays": steps,
            "matches_eager": bool(same), "settle": settled,
            "note": "prepare + score + top-K captured once as a HIP graph and replayed; wall-clock between "
                    "synchronisations like the headline"}


def pipelined_leg(L, ctx_a, ctx_b, hidden, pos, q, w, comp_k, B, N, ref_scores, ref_mask, steps: int,
                  settle_s: float, beside: str = "prepare") -> dict:
    """Consecutive passes pipelined over two streams: the query preparation
    and the score of pass i run on the current stream with context ctx_a,
    its top-K on a second stream with context ctx_b (each context serves one
    stream).  beside="prepare": pass i's top-K starts when its score ends,
    beside pass i+1's query preparation; beside="score": it starts when pass
    i+1's preparation ends, beside pass i+1's score kernel (whose waves leave
    room on each SIMD for a selection wave).  Scores and masks are
    double-buffered; pass i's score waits for the selection that last read
    its buffer (pass i-2).  Every pass does the whole path.  Timed by host
    wall-clock between device synchronisations over `steps` passes, after
    settle_s seconds of passes; the last pass's scores and mask must equal
    the sequential step's (ref_*) bit for bit."""
    import torch

    sa = torch.cuda.current_stream()
    sb = torch.cuda.Stream()
    scores = [torch.empty((B, N), device="cuda") for _ in range(2)]
    masks = [torch.empty((B, N), dtype=torch.bool, device="cuda") for _ in range(2)]
    ev_score = [torch.cuda.Event() for _ in range(2)]
    ev_sel = [torch.cuda.Event() for _ in range(2)]
    ev_prep = torch.cuda.Event()
    for e in ev_sel:
        e.record(sa)
    state = {"i": 0, "pending": None}

    def select(b, after):
        sb.wait_event(after)
        L.fm_select_topk(ctx_b, scores[b], B, N, None, TOP_K, masks[b], sb.cuda_stream)
        ev_sel[b].record(sb)

    def one():
        b = state["i"] & 1
        L.fm_prepare_query(ctx_a, hidden, pos, B, q, w, sa.cuda_stream)
        if beside == "score" and state["pending"] is not None:
            ev_prep.record(sa)
            select(state["pending"], ev_prep)
            state["pending"] = None
        sa.wait_event(ev_sel[b])
        L.fm_score(ctx_a, q, w, comp_k, B, N, None, L.FM_ENSEMBLE_MAX, scores[b], None, sa.cuda_stream)
        ev_score[b].record(sa)
        if beside == "score":
            state["pending"] = b
        else:
            select(b, ev_score[b])
        state["i"] += 1

    def drain():
        if state["pending"] is not None:
            select(state["pending"], ev_score[state["pending"]])
            state["pending"] = None

    def block_step():
        one()

    settled = settle(block_step, sa, settle_s)
    drain()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one()
    drain()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    last = (state["i"] - 1) & 1
    same = bool(torch.equal(scores[last], ref_scores) and torch.equal(masks[last], ref_mask))
    return {"us_per_step": wall * 1e6, "steps": steps, "matches_sequential": same, "settle": settled,
            "beside": beside,
            "note": f"pass i's top-K on a second stream (own context) beside pass i+1's "
                    f"{'query preparation' if beside == 'prepare' else 'score kernel'}; scores and masks "
                    "double-buffered"}


def _parity(ref: dict, gpu_scores, gpu_mask, valid_n: int, top_k, threshold, band: float = 2e-3) -> dict:
    """One row's GPU outputs against the oracle's: the largest score error
    over the valid chunks, and the mask entries that differ, split into
    those whose oracle score lies within `band` of the K-th score (or of the
    threshold) and the others (the acceptance rule allows only the first)."""
    import numpy as np

    s_ref = ref["scores"][:valid_n]
    err = float(np.max(np.abs(gpu_scores[:valid_n].astype(np.float64) - s_ref))) if valid_n else 0.0
    cut = threshold if top_k is None else (np.sort(s_ref)[::-1][min(top_k, valid_n) - 1] if valid_n else 0.0)
    diff = np.asarray(gpu_mask, np.uint8) != ref["mask"]
    near = np.zeros_like(diff)
    near[:valid_n] = np.abs(s_ref - cut) <= band
    return {"max_abs_score_err": err, "mask_diff_in_band": int((diff & near).sum()),
            "mask_diff_outside_band": int((diff & ~near).sum())}


def _merge_parity(acc: dict | None, p: dict) -> dict:
    if acc is None:
        return dict(p, rows=1)
    return {"max_abs_score_err": max(acc["max_abs_score_err"], p["max_abs_score_err"]),
            "mask_diff_in_band": acc["mask_diff_in_band"] + p["mask_diff_in_band"],
            "mask_diff_outside_band": acc["mask_diff_outside_band"] + p["mask_diff_outside_band"],
            "rows": acc["rows"] + 1}


def cpu_baseline(budget_s: float, leg_inputs: dict, config_inputs: dict | None = None,
                 config_budget_s: float = 3.0):
    """The oracle, as it stands, on whole rows of the workload until the time
    budget is spent (at least one row); chunks/s over the rows done.  Also
    times the oracle's resident delta and subset top-K on the host copies of
    the inputs the next-row legs ran on (all B rows each), and, under
    `configs`, whole rows of each other workload on the host copies of the
    inputs its GPU leg ran on (valid chunks only, config_budget_s each)."""
    import numpy as np

    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max((d.get("num_threads", 1) for d in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = 1
    wl = synth.WORKLOADS[WORKLOAD_ID]
    weights = synth.make_weights()
    hidden = synth.make_hidden(wl)
    pos = synth.make_positions(wl)
    cfg = oracle.OracleConfig()
    rows = 0
    elapsed = 0.0
    parity = None
    while rows < wl.batch:
        comp = synth.make_comp_k(wl, rows=[rows])[0]   # generation is outside the timed part
        t1 = time.perf_counter()
        ref = oracle.run_row(weights, hidden[rows], int(pos[rows]), comp, cfg, mode="max", top_k=TOP_K)
        elapsed += time.perf_counter() - t1
        if "headline" in leg_inputs:
            g_scores, g_mask = leg_inputs["headline"]
            parity = _merge_parity(parity, _parity(ref, g_scores[rows], g_mask[rows], wl.n_chunks, TOP_K, None))
        rows += 1
        if elapsed >= budget_s:
            break
    next_rows = {}
    if "resident_delta" in leg_inputs:
        cur, prev = leg_inputs["resident_delta"]
        t1 = time.perf_counter()
        for b in range(cur.shape[0]):
            oracle.resident_delta(cur[b], prev[b])
        next_rows["resident_delta_us"] = (time.perf_counter() - t1) * 1e6
    if "subset_topk" in leg_inputs:
        step, sub = leg_inputs["subset_topk"]
        t1 = time.perf_counter()
        for b in range(step.shape[0]):
            oracle.select_topk_subset(step[b], sub[b], TOP_K)
        next_rows["subset_topk_us"] = (time.perf_counter() - t1) * 1e6
    configs = {}
    for cid, inp in (config_inputs or {}).items():
        cwl = synth.WORKLOADS[cid]
        ccfg = oracle.OracleConfig(yarn_factor=cwl.yarn_factor, yarn_orig_ctx=cwl.yarn_orig_ctx,
                                   yarn_beta_fast=cwl.yarn_beta_fast, yarn_beta_slow=cwl.yarn_beta_slow)
        done = chunks = 0
        spent = 0.0
        cpar = None
        while done < cwl.batch:
            vn = int(inp["valid_n"][done])
            t1 = time.perf_counter()
            ref = oracle.run_row(weights, inp["hidden"][done], int(inp["positions"][done]), inp["comp_k"][done],
                                 ccfg, valid_n=vn, mode=cwl.mode, top_k=cwl.top_k, threshold=cwl.threshold)
            spent += time.perf_counter() - t1
            cpar = _merge_parity(cpar, _parity(ref, inp["scores"][done], inp["mask"][done], vn, cwl.top_k,
                                               cwl.threshold))
            done += 1
            chunks += vn
            if spent >= config_budget_s:
                break
        configs[cwl.name] = {"value": chunks / spent, "unit": "chunks/s", "rows": done, "valid_chunks": chunks,
                             "seconds": spent, "parity": cpar}
    return {"value": rows * wl.n_chunks / elapsed, "unit": "chunks/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{rows} of {wl.batch} rows x {wl.n_chunks} chunks (query prep, 3-layer score, max "
                      f"ensemble, top-{TOP_K}), fp64 numpy, {elapsed:.1f} s",
            "parity": parity, "next_rows": next_rows, "configs": configs, "_cpu_model": _cpu_model()}


def resident_delta_leg(L, r, hidden, pos, comp_k, q, w, mask, B, N, sh, stream, steps, leg_inputs):
    """fm_resident_delta on this step's top-K mask against the previous
    cycle's: HIP-event time per call on the launch stream and algorithmic HBM
    bytes (both masks read, the three index lists and counts written).  Host
    copies of the two masks go into leg_inputs for the CPU baseline."""
    import numpy as np
    import torch

    qp = torch.empty_like(q)
    wp = torch.empty_like(w)
    sp = torch.empty((B, N), device="cuda")
    prev = torch.empty_like(mask)
    L.fm_prepare_query(r.ctx, hidden, pos - 256, B, qp, wp, sh)
    L.fm_score(r.ctx, qp, wp, comp_k, B, N, None, L.FM_ENSEMBLE_MAX, sp, None, sh)
    L.fm_select_topk(r.ctx, sp, B, N, None, TOP_K, prev, sh)
    cap = TOP_K
    lists = [torch.empty((B, cap), dtype=torch.int32, device="cuda") for _ in range(3)]
    counts = [torch.empty((B,), dtype=torch.int32, device="cuda") for _ in range(3)]

    def call():
        L.fm_resident_delta(r.ctx, prev, mask, B, N, cap, lists[0], counts[0], lists[1], counts[1], lists[2],
                            counts[2], sh)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    ev = [TimingEvent() for _ in range(2)]
    ev[0].record(stream)
    for _ in range(steps):
        call()
    ev[1].record(stream)
    torch.cuda.synchronize()
    t = ev[0].elapsed_time(ev[1]) * 1e-3 / steps
    n = [c.cpu().numpy().astype(np.int64) for c in counts]
    nbytes = 2 * B * N + 4 * int(n[0].sum() + n[1].sum() + n[2].sum()) + 3 * 4 * B
    leg_inputs["resident_delta"] = (mask.cpu().numpy(), prev.cpu().numpy())
    return {"us": t * 1e6, "hbm_gbs": nbytes / t / 1e9, "hbm_frac": nbytes / t / 1e9 / PEAK_HBM_GBS,
            "bytes": nbytes, "resident_per_row": float(n[0].mean()), "entering_per_row": float(n[1].mean()),
            "leaving_per_row": float(n[2].mean())}


def variants_leg(L, r, q, w, comp_k, scores, mask, B, N, sh, stream, steps):
    """The same workload's other ensemble and selection modes (mean ensemble
    with top-512, max ensemble with the 0.5 threshold by fm_score_threshold,
    and the same threshold by fm_score + fm_select_threshold), score + select
    per call pair from HIP events on the launch stream (median): launched in
    turn, so all see the same thermal state."""
    import numpy as np
    import torch

    def mean_topk():
        L.fm_score(r.ctx, q, w, comp_k, B, N, None, L.FM_ENSEMBLE_MEAN, scores, None, sh)
        L.fm_select_topk(r.ctx, scores, B, N, None, TOP_K, mask, sh)

    def max_threshold():
        L.fm_score_threshold(r.ctx, q, w, comp_k, B, N, None, L.FM_ENSEMBLE_MAX, 0.5, scores, mask, None, sh)

    def max_threshold_separate():
        L.fm_score(r.ctx, q, w, comp_k, B, N, None, L.FM_ENSEMBLE_MAX, scores, None, sh)
        L.fm_select_threshold(r.ctx, scores, B, N, None, 0.5, mask, sh)

    def max_topk():
        L.fm_score(r.ctx, q, w, comp_k, B, N, None, L.FM_ENSEMBLE_MAX, scores, None, sh)
        L.fm_select_topk(r.ctx, scores, B, N, None, TOP_K, mask, sh)

    fns = (("max_top512", max_topk), ("mean_top512", mean_topk), ("max_threshold_0.5", max_threshold),
           ("max_threshold_0.5_separate_calls", max_threshold_separate))
    for _, fn in fns:
        fn()
    torch.cuda.synchronize()
    ev = []
    n = max(1, steps // 5)
    for _ in range(n):
        for name, fn in fns:
            e = [TimingEvent() for _ in range(2)]
            e[0].record(stream)
            fn()
            e[1].record(stream)
            ev.append((name, e))
    torch.cuda.synchronize()
    out = {}
    for name, _ in fns:
        t = float(np.median([e[0].elapsed_time(e[1]) for nm, e in ev if nm == name])) * 1e-3
        out[name] = {"score_select_us": t * 1e6, "chunks_per_s": B * N / t}
    out["calls_each"] = n
    return out


def score_fp8_leg(L, r, q, w, comp_k, scores, B, N, sh, stream, steps):
    """fm_score_fp8 on the same prepared queries, launched alternately with
    fm_score (f16) so both see the same thermal state; HIP-event times per
    call and per score-kernel launch on the launch stream (median, p10, p90
    of the calls; the rates use the launch).  The method's 49152 flop
    per chunk are priced against the fp8 MFMA peak; the MFMA work it issues
    (two e4m3 query parts per head, plus the linear-term fragment: 102400
    flop per chunk) is reported beside it."""
    import numpy as np
    import torch

    fns = (("f16", L.fm_score), ("fp8", L.fm_score_fp8))
    for _ in range(3):
        for _, fn in fns:
            fn(r.ctx, q, w, comp_k, B, N, None, L.FM_ENSEMBLE_MAX, scores, None, sh)
    torch.cuda.synchronize()
    ev = []
    for _ in range(steps):
        for name, fn in fns:
            e = [TimingEvent() for _ in range(4)]
            e[0].record(stream)
            L.fm_set_score_events(r.ctx, e[2].ev, e[3].ev)  # the score kernel's launch alone
            fn(r.ctx, q, w, comp_k, B, N, None, L.FM_ENSEMBLE_MAX, scores, None, sh)
            L.fm_set_score_events(r.ctx, None, None)
            e[1].record(stream)
            ev.append((name, e))
    torch.cuda.synchronize()
    t = {"f16": [], "fp8": []}
    tk = {"f16": [], "fp8": []}
    for name, e in ev:
        t[name].append(e[0].elapsed_time(e[1]) * 1e-3)
        tk[name].append(e[2].elapsed_time(e[3]) * 1e-3)
    t8 = float(np.median(t["fp8"]))
    t16 = float(np.median(t["f16"]))
    k8 = float(np.median(tk["fp8"]))
    k16 = float(np.median(tk["f16"]))
    chunks = B * N
    achieved = FLOP_PER_CHUNK * chunks / k8 / 1e12
    issued = (2 * FLOP_PER_CHUNK + 16 * 128 * 2) * chunks / k8 / 1e12
    return {"us": t8 * 1e6, "us_p10": float(np.percentile(t["fp8"], 10)) * 1e6,
            "us_p90": float(np.percentile(t["fp8"], 90)) * 1e6, "f16_us_same_run": t16 * 1e6,
            "kernel_us": k8 * 1e6, "f16_kernel_us_same_run": k16 * 1e6,
            "speed_vs_f16": t16 / t8, "kernel_speed_vs_f16": k16 / k8, "chunks_per_s": chunks / t8,
            "achieved_tflops": achieved, "peak_tflops": PEAK_FP8_TFLOPS, "frac": achieved / PEAK_FP8_TFLOPS,
            "issued_mfma_tflops": issued, "issued_frac": issued / PEAK_FP8_TFLOPS,
            "hbm_gbs": SCORE_BYTES_PER_CHUNK * chunks / k8 / 1e9,
            "hbm_frac": SCORE_BYTES_PER_CHUNK * chunks / k8 / 1e9 / PEAK_HBM_GBS,
            "rates_from": "the score kernel's launch alone (events libfm records around it); 'us' is the whole call"}


def subset_topk_leg(L, r, scores, B, N, sh, stream, steps, leg_inputs, resident_k=32768, key="subset_topk"):
    """fm_select_topk_subset: a decode step's top-512 within each row's
    resident set.  The resident set is this pass's top-`resident_k` chunks per
    row (32768 = 12.5% of N, the share of the compressed cache the model card
    keeps on the GPU; 8192 is that share of a 256K-token context's 65536
    chunks, and takes the one-launch short-list path); the step's scores are
    seeded uniform stand-ins (the pages do not define the step's score
    function).  HIP-event time per call on the launch stream; bytes = the
    list and the gathered scores (4 B each per entry) plus the chosen
    indices.  Host copies of the step's scores and the lists go into
    leg_inputs[key] for the CPU baseline (key None: not kept)."""
    import torch

    keep = torch.empty((B, N), dtype=torch.bool, device="cuda")
    L.fm_select_topk(r.ctx, scores, B, N, None, resident_k, keep, sh)
    sub = torch.empty((B, resident_k), dtype=torch.int32, device="cuda")
    n_sub = torch.empty((B,), dtype=torch.int32, device="cuda")
    L.fm_resident_delta(r.ctx, None, keep, B, N, resident_k, sub, n_sub, None, None, None, None, sh)
    g = torch.Generator().manual_seed(77)
    step = torch.rand((B, N), generator=g).cuda()
    out = torch.empty((B, TOP_K), dtype=torch.int32, device="cuda")
    n_out = torch.empty((B,), dtype=torch.int32, device="cuda")

    def call():
        L.fm_select_topk_subset(r.ctx, step, B, N, sub, n_sub, resident_k, TOP_K, out, n_out, sh)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    ev = [TimingEvent() for _ in range(2)]
    ev[0].record(stream)
    for _ in range(steps):
        call()
    ev[1].record(stream)
    torch.cuda.synchronize()
    t = ev[0].elapsed_time(ev[1]) * 1e-3 / steps
    nbytes = B * (8 * resident_k + 4 * TOP_K + 8)
    if key is not None:
        leg_inputs[key] = (step.cpu().numpy(), sub.cpu().numpy())
    return {"us": t * 1e6, "resident_per_row": resident_k, "top_k": TOP_K, "entries_per_s": B * resident_k / t,
            "bytes": nbytes, "hbm_gbs": nbytes / t / 1e9}


def mask_logits_leg(L, r, mask, B, N, sh, stream, steps, heads=64):
    """fm_mask_logits: this step's top-512 keep mask applied to bf16 attention
    logits [B, 64 heads, N] in place (synthetic values).  HIP-event time per
    call on the launch stream; algorithmic bytes per call = the mask, plus per
    (row, head) 16-byte vector of 8 chunks: nothing when all are kept, one
    write when none is, a read and a write when some are."""
    import numpy as np
    import torch

    logits = torch.empty((B, heads, N), dtype=torch.bfloat16, device="cuda")
    logits.normal_(generator=torch.Generator(device="cuda").manual_seed(5))

    def call():
        L.fm_mask_logits(r.ctx, logits, L.FM_DTYPE_BF16, B, heads, N, mask, sh)

    for _ in range(2):
        call()
    torch.cuda.synchronize()
    ev = [TimingEvent() for _ in range(2)]
    ev[0].record(stream)
    for _ in range(steps):
        call()
    ev[1].record(stream)
    torch.cuda.synchronize()
    t = ev[0].elapsed_time(ev[1]) * 1e-3 / steps
    m = mask.cpu().numpy().astype(bool)
    V = 8  # bf16 chunks per 16-byte vector
    full = (N // V) * V
    g = m[:, :full].reshape(B, -1, V).sum(axis=2)
    none_kept, mixed = int((g == 0).sum()), int(((g > 0) & (g < V)).sum())
    nbytes = B * N + heads * 16 * (none_kept + 2 * mixed)
    del logits
    return {"us": t * 1e6, "heads": heads, "dtype": "bf16", "bytes": nbytes, "hbm_gbs": nbytes / t / 1e9,
            "hbm_frac": nbytes / t / 1e9 / PEAK_HBM_GBS}


def config_leg(cid: int, weights_dev, steps: int, settle_s: float, config_inputs: dict, flush_bytes: int = 1 << 29):
    """One of the other seeded workloads on its own context: the whole pass
    (fm_prepare_query, then fm_score + fm_select_topk, or fm_score_threshold,
    with the workload's ensemble and selection, valid_n for ragged rows)
    timed like the headline (settle, then `steps` back-to-back steps between two HIP events), plus
    per-phase events on a second run of `steps` steps (medians), the score kernel's own launch
    among them (the score rates use it).  Workloads
    whose inputs fit the 256 MB Infinity Cache (B=1 N=4096, B=8 N=65536) are
    also timed flushed: a 512 MB device fill before each step evicts it, and
    events bracket the step alone.  Rates count valid chunks only.  The
    planted workload plants along the queries fm_prepare_query returns for
    its rows (the tests plant along the oracle's; the two agree to about
    1e-6).  Host copies of the inputs go into config_inputs[cid] for the CPU
    baseline."""
    import numpy as np
    import torch

    import synth
    import sparse_attention_chunk_amd as fm

    wl = synth.WORKLOADS[cid]
    B, N = wl.batch, wl.n_chunks
    L = fm._lib
    yarn = None
    if wl.yarn_factor != 1.0:
        yarn = {"factor": wl.yarn_factor, "orig_ctx": wl.yarn_orig_ctx, "beta_fast": wl.yarn_beta_fast,
                "beta_slow": wl.yarn_beta_slow}
    r = fm.FlashMemoryRetriever(weights_dev, max_batch=B, max_n=N, yarn=yarn)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    hidden_np, pos_np, vn_np = synth.make_hidden(wl), synth.make_positions(wl), synth.make_valid_n(wl)
    hidden = torch.from_numpy(hidden_np).cuda()
    pos = torch.from_numpy(pos_np).cuda()
    q = torch.empty((3, B, 64, 128), device="cuda")
    w = torch.empty((3, B, 64), device="cuda")
    dirs = None
    if wl.plant_fraction > 0:
        L.fm_prepare_query(r.ctx, hidden, pos, B, q, w, sh)
        qh = q.cpu().numpy()
        dirs = {b: qh[:, b] for b in range(B)}
    comp_np = synth.make_comp_k(wl, plant_dirs=dirs)
    comp_k = torch.from_numpy(comp_np).cuda()
    valid_n = torch.from_numpy(vn_np).cuda() if wl.ragged else None
    scores = torch.empty((B, N), device="cuda")
    mask = torch.empty((B, N), dtype=torch.bool, device="cuda")
    mode = L.FM_ENSEMBLE_MEAN if wl.mode == "mean" else L.FM_ENSEMBLE_MAX
    valid = int(vn_np.astype(np.int64).sum())

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        L.fm_prepare_query(r.ctx, hidden, pos, B, q, w, sh)
        if ev is not None:
            ev[1].record(stream)
            L.fm_set_score_events(r.ctx, ev[4].ev, ev[5].ev)  # the score kernel's launch alone
        if wl.top_k is not None:
            L.fm_score(r.ctx, q, w, comp_k, B, N, valid_n, mode, scores, None, sh)
        else:
            L.fm_score_threshold(r.ctx, q, w, comp_k, B, N, valid_n, mode, wl.threshold, scores, mask, None, sh)
        if ev is not None:
            L.fm_set_score_events(r.ctx, None, None)
            ev[2].record(stream)
        if wl.top_k is not None:
            L.fm_select_topk(r.ctx, scores, B, N, valid_n, wl.top_k, mask, sh)
        if ev is not None:
            ev[3].record(stream)

    step()
    torch.cuda.synchronize()
    st = settle(step, stream, settle_s)
    ends = [TimingEvent(), TimingEvent()]
    ends[0].record(stream)
    for _ in range(steps):
        step()
    ends[1].record(stream)
    torch.cuda.synchronize()
    t_step = ends[0].elapsed_time(ends[1]) * 1e-3 / steps
    evs = [[TimingEvent() for _ in range(6)] for _ in range(steps)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    ph = np.array([[e[i].elapsed_time(e[i + 1]) * 1e-3 for i in range(3)] for e in evs])
    t_prep, t_score, t_sel = (float(np.median(ph[:, i])) for i in range(3))
    t_kern = float(np.median([e[4].elapsed_time(e[5]) * 1e-3 for e in evs]))
    out = {
        "workload": wl.name, "batch": B, "n_chunks": N, "valid_chunks": valid,
        "ensemble": wl.mode, "select": f"top-{wl.top_k}" if wl.top_k is not None else f"threshold {wl.threshold}",
        "step_us": t_step * 1e6, "step_chunks_per_s": valid / t_step,
        "chunks_per_s": valid / (t_score + t_sel),
        "breakdown_us": {"prepare_query": t_prep * 1e6, "score": t_score * 1e6, "select": t_sel * 1e6,
                         "score_kernel": t_kern * 1e6},
        "score_tflops": FLOP_PER_CHUNK * valid / t_kern / 1e12,
        "score_mfma_frac": FLOP_PER_CHUNK * valid / t_kern / 1e12 / PEAK_F16_TFLOPS,
        "score_hbm_gbs": SCORE_BYTES_PER_CHUNK * valid / t_kern / 1e9,
        "score_hbm_frac": SCORE_BYTES_PER_CHUNK * valid / t_kern / 1e9 / PEAK_HBM_GBS,
        "score_rates_from": "the score kernel's launch alone (events libfm records around it); 'score' in "
                            "breakdown_us is the whole call (packing, ragged-row planning, -inf tail and kernel)",
        "select_hbm_gbs": 5 * valid / t_sel / 1e9,
        "prepare_hbm_gbs": QUERY_WEIGHT_BYTES / t_prep / 1e9,
        "settle": st,
    }
    if comp_np.nbytes + QUERY_WEIGHT_BYTES < (256 << 20):
        junk = torch.empty(flush_bytes // 4, device="cuda")
        fl = []
        for i in range(steps):
            junk.fill_(float(i))
            e = [TimingEvent(), TimingEvent()]
            e[0].record(stream)
            step()
            e[1].record(stream)
            fl.append(e)
        torch.cuda.synchronize()
        t_fl = float(np.median([e[0].elapsed_time(e[1]) for e in fl])) * 1e-3
        out["flushed"] = {"step_us": t_fl * 1e6, "step_chunks_per_s": valid / t_fl,
                          "note": "512 MB device fill before each step evicts the Infinity Cache; events "
                                  "bracket the step alone (median)"}
        del junk
    step()
    config_inputs[cid] = {"hidden": hidden_np, "positions": pos_np, "valid_n": vn_np, "comp_k": comp_np,
                          "scores": scores.cpu().numpy(), "mask": mask.cpu().numpy()}
    r.close()
    del comp_k
    torch.cuda.empty_cache()
    return out


def _rocm_version() -> str:
    try:
        with open("/opt/rocm/.info/version") as f:
            return f.read().strip()
    except OSError:
        return "unknown"


def gemm_ceiling_leg(seconds: float = 1.0, n: int = 8192, calls: int = 30):
    """What a vendor-tuned MFMA kernel sustains on this chip under the same
    conditions: a dense 16-bit GEMM (n x n x n, fp32 accumulation) through
    torch.matmul, i.e. ROCm's BLAS, in f16 and in bf16 (whose library kernels
    are the faster here).  For each type the calls run back to back for
    `seconds` first, so that the chip has reached the clock its power limit
    allows, then `calls` more are timed between two synchronisations.
    `tflops` is the faster type's.  A context for the roofline fraction, not
    a part of the scoring pass."""
    import torch

    res = {}
    for name, dt_ in (("f16", torch.float16), ("bf16", torch.bfloat16)):
        a = torch.randn(n, n, device="cuda", dtype=dt_)
        b = torch.randn(n, n, device="cuda", dtype=dt_)
        c = torch.empty(n, n, device="cuda", dtype=dt_)
        t0 = time.perf_counter()
        settle = 0
        while time.perf_counter() - t0 < seconds:
            for _ in range(10):
                torch.matmul(a, b, out=c)
            torch.cuda.synchronize()
            settle += 10
        t0 = time.perf_counter()
        for _ in range(calls):
            torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / calls
        del a, b, c
        torch.cuda.empty_cache()
        res[name] = {"us_per_call": dt * 1e6, "tflops": 2.0 * n ** 3 / dt / 1e12, "settle_calls": settle}
    best = max(res.values(), key=lambda r: r["tflops"])["tflops"]
    return {"what": f"dense {n}x{n}x{n} GEMM (fp32 accumulation) through torch.matmul (ROCm BLAS), f16 and bf16, "
                    f"each timed after a second of back-to-back calls",
            **res, "tflops": best, "frac_of_peak": best / PEAK_F16_TFLOPS}


def _cpu_model() -> str:
    """The host's CPU model name as /proc/cpuinfo gives it (a virtual machine
    may report only the family) and the logical CPUs this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{model}, {len(os.sched_getaffinity(0))} logical CPUs available"


def main(argv=None):
    args = parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the scoring pass is built and timed on a single MI355X; "
              "--gpus above 1 is not supported.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import synth
    import sparse_attention_chunk_amd as fm

    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = 1 << 28  # 1 GiB of float32
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": 4 * n, "copies": 3}))
        return 0

    wl = synth.WORKLOADS[WORKLOAD_ID]
    B, N = wl.batch, wl.n_chunks
    t_gen = time.perf_counter()
    weights = fm.weights_to_device(synth.make_weights())
    hidden = torch.from_numpy(synth.make_hidden(wl)).cuda()
    pos = torch.from_numpy(synth.make_positions(wl)).cuda()
    comp_k = torch.from_numpy(synth.make_comp_k(wl)).cuda()
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    print(f"# inputs ready in {t_gen:.1f} s: comp_k {tuple(comp_k.shape)}", file=sys.stderr, flush=True)

    r = fm.FlashMemoryRetriever(weights, max_batch=B, max_n=N)
    q = torch.empty((3, B, 64, 128), device="cuda")
    w = torch.empty((3, B, 64), device="cuda")
    scores = torch.empty((B, N), device="cuda")
    mask = torch.empty((B, N), dtype=torch.bool, device="cuda")
    L = fm._lib
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        L.fm_prepare_query(r.ctx, hidden, pos, B, q, w, sh)
        if ev is not None:
            ev[1].record(stream)
            L.fm_set_score_events(r.ctx, ev[4].ev, ev[5].ev)  # the score kernel's launch alone
        L.fm_score(r.ctx, q, w, comp_k, B, N, None, L.FM_ENSEMBLE_MAX, scores, None, sh)
        if ev is not None:
            L.fm_set_score_events(r.ctx, None, None)
            ev[2].record(stream)
        L.fm_select_topk(r.ctx, scores, B, N, None, TOP_K, mask, sh)
        if ev is not None:
            ev[3].record(stream)

    # The next rows of the path and the workload's other modes, each timed on
    # its own with HIP events, run before the warmup: the chip takes a few
    # tens of steps of load after idle to reach its steady clock, so the
    # timed steps start at that clock whatever W is (run right before the
    # timed steps instead, the legs' own load left them about 1.5% slower).
    # Their inputs are this pass's outputs: one step (not timed) makes them.
    # The resident delta compares this cycle's mask with the previous
    # cycle's (the same pass for the decode token 64 steps earlier:
    # positions - 256 at 4 tokens per chunk).  The variants leg overwrites
    # scores and mask, so it runs last.
    step()
    leg_inputs = {}
    resident = resident_delta_leg(L, r, hidden, pos, comp_k, q, w, mask, B, N, sh, stream, args.steps, leg_inputs)
    score_fp8 = score_fp8_leg(L, r, q, w, comp_k, torch.empty_like(scores), B, N, sh, stream, args.steps)
    subset = subset_topk_leg(L, r, scores, B, N, sh, stream, args.steps, leg_inputs)
    subset_short = subset_topk_leg(L, r, scores, B, N, sh, stream, args.steps, leg_inputs, resident_k=8192, key=None)
    masking = mask_logits_leg(L, r, mask, B, N, sh, stream, args.steps)
    variants = variants_leg(L, r, q, w, comp_k, scores, mask, B, N, sh, stream, args.steps)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Back-to-back load right before the timed steps, whatever W is: after the
    # legs' host work the chip idles briefly and lowers its clock again.  The
    # firmware's clock and power figures are sampled over this phase (not
    # over the timed steps, which the sampling thread would perturb).
    clocks = ClockSampler().start()
    settled = settle(step, stream, args.settle_seconds)
    clocks.stop()

    # Per-phase HIP events on every EVENT_STRIDE-th timed step: each record
    # still costs the stream about 1 us, so recording four on every step would
    # slow the loop being timed by about 1%.
    events = [[TimingEvent() for _ in range(6)] if i % EVENT_STRIDE == 0 else None
              for i in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    timed = [e for e in events if e is not None]
    prep = np.array([e[0].elapsed_time(e[1]) for e in timed]) * 1e-3
    score = np.array([e[1].elapsed_time(e[2]) for e in timed]) * 1e-3
    sel = np.array([e[2].elapsed_time(e[3]) for e in timed]) * 1e-3
    kern = np.array([e[4].elapsed_time(e[5]) for e in timed]) * 1e-3
    s_step = wall / args.steps
    chunks = B * N
    t_score = float(score.mean())
    t_kern = float(kern.mean())
    achieved = FLOP_PER_CHUNK * chunks / t_kern / 1e12
    traffic = read_traffic(chunks)
    leg_inputs["headline"] = (scores.cpu().numpy(), mask.cpu().numpy())

    def step_body(h):
        L.fm_prepare_query(r.ctx, hidden, pos, B, q, w, h)
        L.fm_score(r.ctx, q, w, comp_k, B, N, None, L.FM_ENSEMBLE_MAX, scores, None, h)
        L.fm_select_topk(r.ctx, scores, B, N, None, TOP_K, mask, h)

    # Supplementary legs after the headline's figures are taken: a failure is
    # reported in their field (the headline line is still printed).
    graph = None
    if not args.no_graph:
        try:
            graph = graph_step_leg(step_body, (q, w, scores, mask), args.steps, args.settle_seconds)
        except Exception as exc:  # noqa: BLE001
            graph = {"error": f"{type(exc).__name__}: {exc}"}
    pipelined = None
    if not args.no_pipelined:
        r_sel = fm.FlashMemoryRetriever(weights, max_batch=B, max_n=N)
        try:
            pipelined = {beside: pipelined_leg(L, r.ctx, r_sel.ctx, hidden, pos, q, w, comp_k, B, N, scores, mask,
                                               args.steps, args.settle_seconds, beside)
                         for beside in ("prepare", "score")}
        except Exception as exc:  # noqa: BLE001
            pipelined = {"error": f"{type(exc).__name__}: {exc}"}
        r_sel.close()
    r.close()
    del comp_k
    torch.cuda.empty_cache()
    configs = {}
    config_inputs = {}
    if not args.no_configs:
        for cid in (1, 2, 3, 4):
            print(f"# workload {cid}: {synth.WORKLOADS[cid].name}", file=sys.stderr, flush=True)
            configs[synth.WORKLOADS[cid].name] = config_leg(cid, weights, args.steps, 0.5, config_inputs)
    ceiling = None
    if not args.no_gemm_ceiling:
        print("# dense 16-bit GEMM ceiling", file=sys.stderr, flush=True)
        ceiling = gemm_ceiling_leg()
        ceiling["score_kernel_frac_of_it"] = achieved / ceiling["tflops"]
    print("# cpu baseline", file=sys.stderr, flush=True)
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.cpu_seconds, leg_inputs, config_inputs)
    cpu_model = cpu.pop("_cpu_model") if cpu else None

    out = {
        "metric": METRIC,
        "value": chunks / s_step,
        "unit": "chunks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": s_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "n_chunks": N, "layers": 3, "heads": 64, "head_dim": 128,
                   "q_lora_rank": 1024, "hidden": 4096, "ensemble": "max", "top_k": TOP_K, "positions": 4 * N},
        "roofline": {
            "kernel": "score_kernel (fused 3-layer score and max ensemble), its launch alone",
            "us_per_launch": t_kern * 1e6,
            "fm_score_call_us": t_score * 1e6,
            "fm_score_call_frac": FLOP_PER_CHUNK * chunks / t_score / 1e12 / PEAK_F16_TFLOPS,
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_F16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_F16_TFLOPS,
            "traffic": traffic,
            "hbm_algorithmic_gbs": SCORE_BYTES_PER_CHUNK * chunks / t_kern / 1e9,
            "hbm_frac": SCORE_BYTES_PER_CHUNK * chunks / t_kern / 1e9 / PEAK_HBM_GBS,
        },
        "mfma_ceiling": ceiling,
        "frac_at_sampled_clock": _frac_at_clock(achieved, clocks.summary()),
        "cpu_baseline": cpu,
        "breakdown_steps": f"HIP events on {len(timed)} of the {args.steps} timed steps (every {EVENT_STRIDE}th)",
        "breakdown_us": {"prepare_query": float(prep.mean() * 1e6), "score": t_score * 1e6,
                         "select_topk": float(sel.mean() * 1e6),
                         "score_kernel": t_kern * 1e6,
                         "score_kernel_median": float(np.median(kern) * 1e6),
                         "prepare_query_median": float(np.median(prep) * 1e6),
                         "score_median": float(np.median(score) * 1e6),
                         "select_topk_median": float(np.median(sel) * 1e6),
                         "score_p10": float(np.percentile(score, 10) * 1e6),
                         "score_p90": float(np.percentile(score, 90) * 1e6)},
        "score_only_chunks_per_s": chunks / t_score,
        # the metric's own definition: valid chunks / (score + select), query prep apart
        "score_select_chunks_per_s": chunks / (t_score + float(sel.mean())),
        "next_rows": {"resident_delta": resident, "score_fp8": score_fp8, "subset_topk": subset,
                      "subset_topk_8192": subset_short,
                      "mask_logits": masking},
        "graph_step": graph,
        "pipelined_step": pipelined,
        "workload_variants": variants,
        "settle": dict(settled, note="untimed back-to-back steps after the warmup, before the timed steps"),
        "clocks": clocks.summary(),
        "configs": configs,
        "host_cpu": cpu_model,
        "software": {"rocm": _rocm_version(), "torch": torch.__version__},
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
