"""Shared helpers for the GPU tests: oracle runs on workload subsets and the
acceptance checks (score tolerance, mask agreement outside the band around
the K-th score or the threshold, and exact self-consistency of the GPU
selection on its own scores)."""

from __future__ import annotations

import json
import os

import numpy as np

import oracle
import synth

SCORE_TOL = 2e-3   # |GPU - oracle| on every per-layer and ensemble score
BAND = 2e-3        # mask disagreement allowed only this close to the K-th score / threshold
Q_TOL = 1e-4       # prepared q, absolute (diagnostic)
W_TOL = 1e-6       # prepared w, absolute (diagnostic)

REPORT = os.environ.get("FM_PARITY_REPORT")  # JSON-lines file for the measured margins, if set


def report(case: str, **vals):
    """Print the measured margins of a case and append them to the file named
    by FM_PARITY_REPORT when it is set."""
    print(case, vals, flush=True)
    if REPORT:
        with open(REPORT, "a") as f:
            f.write(json.dumps({"case": case, **{k: float(v) for k, v in vals.items()}}) + "\n")


def oracle_config(wl: synth.Workload) -> oracle.OracleConfig:
    return oracle.OracleConfig(yarn_factor=wl.yarn_factor, yarn_orig_ctx=wl.yarn_orig_ctx,
                               yarn_beta_fast=wl.yarn_beta_fast, yarn_beta_slow=wl.yarn_beta_slow)


def yarn_kwargs(wl: synth.Workload):
    if wl.yarn_factor == 1.0:
        return None
    return {"factor": wl.yarn_factor, "orig_ctx": wl.yarn_orig_ctx, "beta_fast": wl.yarn_beta_fast,
            "beta_slow": wl.yarn_beta_slow}


def subset_inputs(wl: synth.Workload, rows, weights_np, plant=True):
    """hidden, positions, valid_n, comp_k and the oracle's q, w for a row subset."""
    rows = list(rows)
    hidden = synth.make_hidden(wl)[rows]
    pos = synth.make_positions(wl)[rows]
    vn = synth.make_valid_n(wl)[rows]
    q, w = oracle.prepare_query(weights_np, hidden, pos, oracle_config(wl))
    dirs = None
    if wl.plant_fraction > 0 and plant:
        dirs = {b: q[:, i] for i, b in enumerate(rows)}
    comp_k = synth.make_comp_k(wl, rows=rows, plant_dirs=dirs)
    return hidden, pos, vn, comp_k, q, w


def oracle_scores(comp_k, q, w, vn, mode):
    """Per-layer [L, B, N] and ensemble [B, N] scores of the oracle."""
    B, N = comp_k.shape[0], comp_k.shape[1]
    per = np.empty((q.shape[0], B, N))
    ens = np.empty((B, N))
    for b in range(B):
        per[:, b], ens[b] = oracle.score_row(comp_k[b], q[:, b], w[:, b], int(vn[b]), mode)
    return per, ens


def max_score_err(gpu, ref):
    """Largest |gpu - ref| over finite entries; -inf entries must coincide."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.array_equal(np.isneginf(gpu), np.isneginf(ref)), "-inf tail differs"
    fin = np.isfinite(ref)
    assert np.all(np.isfinite(gpu[fin])), "non-finite GPU score"
    return float(np.max(np.abs(gpu[fin] - ref[fin]))) if fin.any() else 0.0


def kth_score(scores_row, vn, k):
    if k <= 0 or k >= vn:
        return None
    return float(np.sort(scores_row[:vn])[::-1][k - 1])


def check_topk(gpu_mask, gpu_scores, ora_scores, vn, k):
    """Exact self-consistency, then agreement with the oracle outside the band.
    Returns the number of band-excused disagreements."""
    gpu_mask = np.asarray(gpu_mask).astype(np.uint8)
    excused = 0
    for b in range(gpu_mask.shape[0]):
        n = int(vn[b])
        own = oracle.select_topk(np.asarray(gpu_scores[b], np.float64), n, k)
        assert np.array_equal(gpu_mask[b], own), f"row {b}: GPU top-{k} is not the top-{k} of its own scores"
        om = oracle.select_topk(ora_scores[b], n, k)
        diff = om != gpu_mask[b]
        kth = kth_score(ora_scores[b], n, k)
        if kth is None:
            assert not diff.any(), f"row {b}: mask differs with no K-th score"
            continue
        band = np.abs(ora_scores[b] - kth) <= BAND
        assert not np.any(diff & ~band), f"row {b}: mask differs outside the band around {kth}"
        excused += int(diff.sum())
    return excused


def check_threshold(gpu_mask, gpu_scores, ora_scores, vn, tau):
    gpu_mask = np.asarray(gpu_mask).astype(np.uint8)
    excused = 0
    for b in range(gpu_mask.shape[0]):
        n = int(vn[b])
        own = oracle.select_threshold(np.asarray(gpu_scores[b], np.float64), n, tau)
        assert np.array_equal(gpu_mask[b], own), f"row {b}: GPU threshold mask is not score > tau"
        om = oracle.select_threshold(ora_scores[b], n, tau)
        diff = om != gpu_mask[b]
        band = np.abs(ora_scores[b] - tau) <= BAND
        assert not np.any(diff & ~band), f"row {b}: threshold mask differs outside the band"
        excused += int(diff.sum())
    return excused
