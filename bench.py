"""Benchmark of the Memory-Indexer scoring pass on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step = the whole pass over one batch: fm_prepare_query (query and weight
branches of the three layers) + fm_score (3-layer fused score, max
ensemble) + fm_select_topk (top-512 per row), on the B=30, N=262144
workload (a 1M-token context at 4x compression, concurrency 30), synthetic
seeded inputs already resident in HBM.  Prints one JSON line.

`roofline` describes the score kernel (the dominant one, MFMA-bound at
49152 flop per chunk); its duration comes from HIP events around each
fm_score call on the stream the kernels run on.  `traffic` is read from the
committed rocprofv3 counter summary when that summary was taken on the
current score-kernel source, else null.  `cpu_baseline` times the fp64
oracle on a bounded sample of the same workload on this host, and under
`next_rows` on the inputs the resident-delta and subset top-K legs ran on.
The next-row and variant legs run before the W warmup and K timed steps.
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
SCORE_SRC = os.path.join(ROOT, "sparse_attention_chunk_amd", "csrc", "fm_score.hip")
PMC_SUMMARY = os.path.join(ROOT, "profiles", "score_kernel_b30_n262144_pmc.txt")


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # The chip takes a few tens of steps after idle to reach its steady clock
    # under this load: five warmup steps time the ramp (about 415 us per step
    # instead of 370 us).
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing (profiling runs)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle time budget for the CPU baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (for scaling FETCH_SIZE/WRITE_SIZE counters)")
    return ap.parse_args(argv)


def source_digest() -> str:
    with open(SCORE_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def read_traffic(chunks_per_launch: int):
    """HBM bytes per score launch from the committed counter summary, or None
    if it is missing or was taken on another version of the score kernel."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    vals = {}
    with open(PMC_SUMMARY) as f:
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


def cpu_baseline(budget_s: float, leg_inputs: dict):
    """The oracle, as it stands, on whole rows of the workload until the time
    budget is spent (at least one row); chunks/s over the rows done.  Also
    times the oracle's resident delta and subset top-K on the host copies of
    the inputs the next-row legs ran on (all B rows each)."""
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
    while rows < wl.batch:
        comp = synth.make_comp_k(wl, rows=[rows])[0]   # generation is outside the timed part
        t1 = time.perf_counter()
        oracle.run_row(weights, hidden[rows], int(pos[rows]), comp, cfg, mode="max", top_k=TOP_K)
        elapsed += time.perf_counter() - t1
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
    return {"value": rows * wl.n_chunks / elapsed, "unit": "chunks/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{rows} of {wl.batch} rows x {wl.n_chunks} chunks (query prep, 3-layer score, max "
                      f"ensemble, top-{TOP_K}), fp64 numpy, {elapsed:.1f} s",
            "next_rows": next_rows, "_cpu_model": _cpu_model()}


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
    with top-512, max ensemble with the 0.5 threshold), score + select per
    call pair from HIP events on the launch stream (median): launched in
    turn, so all see the same thermal state."""
    import numpy as np
    import torch

    def mean_topk():
        L.fm_score(r.ctx, q, w, comp_k, B, N, None, L.FM_ENSEMBLE_MEAN, scores, None, sh)
        L.fm_select_topk(r.ctx, scores, B, N, None, TOP_K, mask, sh)

    def max_threshold():
        L.fm_score(r.ctx, q, w, comp_k, B, N, None, L.FM_ENSEMBLE_MAX, scores, None, sh)
        L.fm_select_threshold(r.ctx, scores, B, N, None, 0.5, mask, sh)

    def max_topk():
        L.fm_score(r.ctx, q, w, comp_k, B, N, None, L.FM_ENSEMBLE_MAX, scores, None, sh)
        L.fm_select_topk(r.ctx, scores, B, N, None, TOP_K, mask, sh)

    fns = (("max_top512", max_topk), ("mean_top512", mean_topk), ("max_threshold_0.5", max_threshold))
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
    call on the launch stream (median, p10, p90).  The method's 49152 flop
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
            e = [TimingEvent() for _ in range(2)]
            e[0].record(stream)
            fn(r.ctx, q, w, comp_k, B, N, None, L.FM_ENSEMBLE_MAX, scores, None, sh)
            e[1].record(stream)
            ev.append((name, e))
    torch.cuda.synchronize()
    t = {"f16": [], "fp8": []}
    for name, e in ev:
        t[name].append(e[0].elapsed_time(e[1]) * 1e-3)
    t8 = float(np.median(t["fp8"]))
    t16 = float(np.median(t["f16"]))
    chunks = B * N
    achieved = FLOP_PER_CHUNK * chunks / t8 / 1e12
    issued = (2 * FLOP_PER_CHUNK + 16 * 128 * 2) * chunks / t8 / 1e12
    return {"us": t8 * 1e6, "us_p10": float(np.percentile(t["fp8"], 10)) * 1e6,
            "us_p90": float(np.percentile(t["fp8"], 90)) * 1e6, "f16_us_same_run": t16 * 1e6,
            "speed_vs_f16": t16 / t8, "chunks_per_s": chunks / t8, "achieved_tflops": achieved,
            "peak_tflops": PEAK_FP8_TFLOPS, "frac": achieved / PEAK_FP8_TFLOPS, "issued_mfma_tflops": issued,
            "issued_frac": issued / PEAK_FP8_TFLOPS, "hbm_gbs": SCORE_BYTES_PER_CHUNK * chunks / t8 / 1e9,
            "hbm_frac": SCORE_BYTES_PER_CHUNK * chunks / t8 / 1e9 / PEAK_HBM_GBS}


def subset_topk_leg(L, r, scores, B, N, sh, stream, steps, leg_inputs, resident_k=32768):
    """fm_select_topk_subset: a decode step's top-512 within each row's
    resident set.  The resident set is this pass's top-32768 chunks per row
    (12.5% of N, the share of the compressed cache the model card keeps on
    the GPU); the step's scores are seeded uniform stand-ins (the pages do
    not define the step's score function).  HIP-event time per call on the
    launch stream; bytes = the list and the gathered scores (4 B each per
    entry) plus the chosen indices.  Host copies of the step's scores and the
    lists go into leg_inputs for the CPU baseline."""
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
    leg_inputs["subset_topk"] = (step.cpu().numpy(), sub.cpu().numpy())
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


def _rocm_version() -> str:
    try:
        with open("/opt/rocm/.info/version") as f:
            return f.read().strip()
    except OSError:
        return "unknown"


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


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
        L.fm_score(r.ctx, q, w, comp_k, B, N, None, L.FM_ENSEMBLE_MAX, scores, None, sh)
        if ev is not None:
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
    masking = mask_logits_leg(L, r, mask, B, N, sh, stream, args.steps)
    variants = variants_leg(L, r, q, w, comp_k, scores, mask, B, N, sh, stream, args.steps)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Per-phase HIP events on every EVENT_STRIDE-th timed step: each record
    # still costs the stream about 1 us, so recording four on every step would
    # slow the loop being timed by about 1%.
    events = [[TimingEvent() for _ in range(4)] if i % EVENT_STRIDE == 0 else None
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
    s_step = wall / args.steps
    chunks = B * N
    t_score = float(score.mean())
    achieved = FLOP_PER_CHUNK * chunks / t_score / 1e12
    traffic = read_traffic(chunks)
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.cpu_seconds, leg_inputs)
    cpu_model = cpu.pop("_cpu_model") if cpu else None
    r.close()

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
            "kernel": "score_kernel (fm_score: q pack + fused 3-layer score)",
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_F16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_F16_TFLOPS,
            "traffic": traffic,
            "hbm_algorithmic_gbs": SCORE_BYTES_PER_CHUNK * chunks / t_score / 1e9,
            "hbm_frac": SCORE_BYTES_PER_CHUNK * chunks / t_score / 1e9 / PEAK_HBM_GBS,
        },
        "cpu_baseline": cpu,
        "breakdown_steps": f"HIP events on {len(timed)} of the {args.steps} timed steps (every {EVENT_STRIDE}th)",
        "breakdown_us": {"prepare_query": float(prep.mean() * 1e6), "score": t_score * 1e6,
                         "select_topk": float(sel.mean() * 1e6),
                         "prepare_query_median": float(np.median(prep) * 1e6),
                         "score_median": float(np.median(score) * 1e6),
                         "select_topk_median": float(np.median(sel) * 1e6),
                         "score_p10": float(np.percentile(score, 10) * 1e6),
                         "score_p90": float(np.percentile(score, 90) * 1e6)},
        "score_only_chunks_per_s": chunks / t_score,
        # the metric's own definition: valid chunks / (score + select), query prep apart
        "score_select_chunks_per_s": chunks / (t_score + float(sel.mean())),
        "next_rows": {"resident_delta": resident, "score_fp8": score_fp8, "subset_topk": subset,
                      "mask_logits": masking},
        "workload_variants": variants,
        "host_cpu": cpu_model,
        "software": {"rocm": _rocm_version(), "torch": torch.__version__},
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
