"""GPU parity against the fp64 oracle, through the C ABI, on every workload.

Scores (per layer and ensemble) within 2e-3 absolute; keep masks identical
outside a 2e-3 band around the oracle's K-th score or the threshold; the GPU
selection exactly the selection of its own scores.  Small workloads and row
subsets are compared element by element; the full-size workload (B=30,
N=262144, the size the benchmark times) on sampled chunks, on full rows, and
by exact self-consistency of every row.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from fm_cases import (BAND, Q_TOL, SCORE_TOL, W_TOL, check_threshold, check_topk, max_score_err, oracle_config,
                      oracle_scores, report, subset_inputs, yarn_kwargs)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def weights_np():
    return synth.make_weights()


@pytest.fixture(scope="module")
def fmmod():
    import sparse_attention_chunk_amd as fm
    return fm


@pytest.fixture(scope="module")
def weights_dev(weights_np, fmmod):
    return fmmod.weights_to_device(weights_np)


@pytest.fixture(scope="module")
def retr(weights_dev, fmmod):
    r = fmmod.FlashMemoryRetriever(weights_dev, max_batch=64, max_n=262144)
    yield r
    r.close()


@pytest.fixture(scope="module")
def retr_yarn(weights_dev, fmmod):
    r = fmmod.FlashMemoryRetriever(weights_dev, max_batch=64, max_n=131072, yarn=yarn_kwargs(synth.WORKLOADS[4]))
    yield r
    r.close()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


# --------------------------------------------------------------------------- query preparation

@pytest.mark.parametrize("cid,rows", [(1, [0]), (3, list(range(8))), (5, [0, 1])])
def test_prepare_query_parity(retr, weights_np, cid, rows):
    wl = synth.WORKLOADS[cid]
    hidden = synth.make_hidden(wl)[rows]
    pos = synth.make_positions(wl)[rows]
    q_ref, w_ref = oracle.prepare_query(weights_np, hidden, pos, oracle_config(wl))
    q, w = retr.prepare_query(dev(hidden), dev(pos))
    dq = np.abs(host(q) - q_ref).max()
    dw = np.abs(host(w) - w_ref).max()
    report(f"prepare_query cfg{cid}", max_abs_q=dq, max_abs_w=dw)
    assert dq <= Q_TOL and dw <= W_TOL


@pytest.mark.parametrize("rows", [list(range(12)), list(range(40))])
def test_prepare_query_parity_yarn(retr_yarn, weights_np, rows):
    """YaRN positions; 40 rows span two groups of 32 batch rows."""
    wl = synth.WORKLOADS[4]
    hidden = synth.make_hidden(wl)[rows]
    pos = synth.make_positions(wl)[rows]
    q_ref, w_ref = oracle.prepare_query(weights_np, hidden, pos, oracle_config(wl))
    q, w = retr_yarn.prepare_query(dev(hidden), dev(pos))
    dq = np.abs(host(q) - q_ref).max()
    dw = np.abs(host(w) - w_ref).max()
    report(f"prepare_query cfg4 yarn B={len(rows)}", max_abs_q=dq, max_abs_w=dw)
    assert dq <= Q_TOL and dw <= W_TOL


@pytest.mark.parametrize("yarn", [False, True])
def test_prepare_query_large_positions(retr, retr_yarn, weights_np, yarn):
    """Positions at the int32 and uint32 edges and past them: the angle in
    double, its reduction to one turn and the float rotation keep q within
    tolerance (the double product position x frequency itself moves by at
    most a few times position x 2^-53 rad between two correct computations:
    about 1e-6 at 2^32)."""
    wl = synth.WORKLOADS[4 if yarn else 3]
    pos = np.array([0, 1, 65535, 65536, 1 << 24, (1 << 31) - 1, 1 << 31, (1 << 32) + 5], np.int64)
    hidden = synth.make_hidden(wl)[:len(pos)]
    q_ref, w_ref = oracle.prepare_query(weights_np, hidden, pos, oracle_config(wl))
    q, w = (retr_yarn if yarn else retr).prepare_query(dev(hidden), dev(pos))
    dq = np.abs(host(q) - q_ref).max()
    dw = np.abs(host(w) - w_ref).max()
    report(f"prepare_query positions up to 2^32 + 5 ({'yarn' if yarn else 'no yarn'})", max_abs_q=dq, max_abs_w=dw)
    assert dq <= Q_TOL and dw <= W_TOL


def test_prepare_query_hidden_magnitudes(retr, weights_np):
    """Hidden rows the activation split must handle: all zero, alternate
    128-wide chunks zero, a single non-zero entry, fp32 subnormal entries,
    and whole rows scaled by 2^-30 and 2^12 (RMSNorm's eps then dominates or
    vanishes).  q is compared absolutely; w, which is not normalised,
    relative to the row's scale."""
    wl = synth.WORKLOADS[3]
    base = synth.make_hidden(wl)[:6].astype(np.float64)
    rows = [np.zeros(4096), base[0].copy(), np.zeros(4096), base[2] * 1e-41, base[3] * 2.0 ** -30, base[4] * 2.0 ** 12]
    rows[1].reshape(32, 128)[::2] = 0.0
    rows[2][1234] = 3.5
    hidden = np.stack(rows).astype(np.float32)
    scale = np.array([1.0, 1.0, 1.0, 1.0, 1.0, 2.0 ** 12])
    pos = synth.make_positions(wl)[:6]
    q_ref, w_ref = oracle.prepare_query(weights_np, hidden.astype(np.float64), pos, oracle_config(wl))
    q, w = retr.prepare_query(dev(hidden), dev(pos))
    q_h, w_h = host(q), host(w)
    assert np.all(np.isfinite(q_h)) and np.all(np.isfinite(w_h))
    assert not np.any(q_h[:, 0]) and not np.any(w_h[:, 0])   # zero row: q = 0, w = 0 exactly
    dq = np.abs(q_h - q_ref).max()
    dw = (np.abs(w_h - w_ref) / scale[None, :, None]).max()
    report("prepare_query hidden magnitudes", max_abs_q=dq, max_w_err_over_scale=dw)
    assert dq <= Q_TOL and dw <= W_TOL


# --------------------------------------------------------------------------- score from oracle queries

@pytest.mark.parametrize("mode", ["max", "mean"])
def test_score_parity_from_oracle_queries(retr, weights_np, mode):
    wl = synth.WORKLOADS[1]
    _, _, vn, comp_k, q, w = subset_inputs(wl, [0], weights_np)
    per_ref, ens_ref = oracle_scores(comp_k, q, w, vn, mode)
    scores, per = retr.score(dev(q.astype(np.float32)), dev(w.astype(np.float32)), dev(comp_k), None, mode,
                             per_layer=True)
    e1 = max_score_err(host(scores), ens_ref)
    e2 = max_score_err(host(per), per_ref)
    report(f"score cfg1 {mode} (oracle q)", max_abs_ens=e1, max_abs_per_layer=e2)
    assert e1 <= SCORE_TOL and e2 <= SCORE_TOL


# --------------------------------------------------------------------------- whole pass per workload

def _whole_pass(r, wl, rows, weights_np, mode, top_k, threshold, use_valid=False):
    hidden, pos, vn, comp_k, q_ref, w_ref = subset_inputs(wl, rows, weights_np)
    per_ref, ens_ref = oracle_scores(comp_k, q_ref, w_ref, vn, mode)
    q, w = r.prepare_query(dev(hidden), dev(pos))
    vdev = dev(vn.astype(np.int32)) if use_valid else None
    scores, per = r.score(q, w, dev(comp_k), vdev, mode, per_layer=True)
    if top_k is not None:
        mask = r.keep_topk(scores, top_k, vdev)
    else:
        mask = r.keep_threshold(scores, threshold, vdev)
    s, p, m = host(scores), host(per), host(mask)
    e_ens = max_score_err(s, ens_ref)
    e_per = max_score_err(p, per_ref)
    if top_k is not None:
        excused = check_topk(m, s, ens_ref, vn, top_k)
    else:
        excused = check_threshold(m, s, ens_ref, vn, threshold)
    return e_ens, e_per, excused


def test_max_batch_whole_pass(retr, weights_np):
    """B = max_batch (64 rows: two groups of 32 in the projections, every wave
    of the score grid on a share of 64 rows): prepared queries and every
    chunk's score against the oracle, each row's top-512 exactly that of its
    own scores and within the band of the oracle's."""
    rng = np.random.default_rng(64)
    B, N = 64, 8192
    hidden = rng.standard_normal((B, 4096)).astype(np.float32)
    pos = rng.integers(0, 1 << 20, B).astype(np.int64)
    comp_k = np.stack([synth.encode_records(rng.standard_normal((N, 128)).astype(np.float32)) for _ in range(B)])
    q_ref, w_ref = oracle.prepare_query(weights_np, hidden, pos, oracle.OracleConfig())
    q, w = retr.prepare_query(dev(hidden), dev(pos))
    dq, dw = np.abs(host(q) - q_ref).max(), np.abs(host(w) - w_ref).max()
    scores = retr.score(q, w, dev(comp_k), None, "max")
    mask = retr.keep_topk(scores, 512)
    s, m = host(scores), host(mask)
    per_ref, ens_ref = oracle_scores(comp_k, q_ref, w_ref, [N] * B, "max")
    e = max_score_err(s, ens_ref)
    exc = check_topk(m, s, ens_ref, [N] * B, 512)
    report(f"max batch B={B} N={N}", max_abs_q=dq, max_abs_w=dw, max_abs_ens=e, band_excused=exc)
    assert dq <= Q_TOL and dw <= W_TOL and e <= SCORE_TOL


def test_cfg1_whole_pass_top512(retr, weights_np):
    e_ens, e_per, exc = _whole_pass(retr, synth.WORKLOADS[1], [0], weights_np, "max", 512, None)
    report("cfg1 b1 n4096 max top512", max_abs_ens=e_ens, max_abs_per_layer=e_per, band_excused=exc)
    assert e_ens <= SCORE_TOL and e_per <= SCORE_TOL


def test_cfg2_planted_top512(retr, weights_np):
    e_ens, e_per, exc = _whole_pass(retr, synth.WORKLOADS[2], [0, 5], weights_np, "max", 512, None)
    report("cfg2 planted rows 0,5 max top512", max_abs_ens=e_ens, max_abs_per_layer=e_per, band_excused=exc)
    assert e_ens <= SCORE_TOL and e_per <= SCORE_TOL


def test_cfg3_mean_threshold(retr, weights_np):
    e_ens, e_per, exc = _whole_pass(retr, synth.WORKLOADS[3], [0, 13, 31], weights_np, "mean", None, 0.5)
    report("cfg3 rows 0,13,31 mean thr0.5", max_abs_ens=e_ens, max_abs_per_layer=e_per, band_excused=exc)
    assert e_ens <= SCORE_TOL and e_per <= SCORE_TOL


def test_cfg4_ragged_yarn_top1024(retr_yarn, weights_np):
    wl = synth.WORKLOADS[4]
    vn_all = synth.make_valid_n(wl)
    rows = sorted({int(np.argmin(vn_all)), int(np.argmax(vn_all)), 7, 30})
    e_ens, e_per, exc = _whole_pass(retr_yarn, wl, rows, weights_np, "max", 1024, None, use_valid=True)
    report("cfg4 ragged yarn max top1024", max_abs_ens=e_ens, max_abs_per_layer=e_per, band_excused=exc)
    assert e_ens <= SCORE_TOL and e_per <= SCORE_TOL


# --------------------------------------------------------------------------- full size, sampled

def test_cfg5_full_size_sampled(retr, weights_np):
    """B=30, N=262144: the benchmark's launch.  Sampled chunks against the
    oracle one by one, two full rows element by element, every row's masks
    self-consistent; also the mean ensemble and the 0.5 threshold on the
    same inputs."""
    wl = synth.WORKLOADS[5]
    B, N = wl.batch, wl.n_chunks
    hidden = synth.make_hidden(wl)
    pos = synth.make_positions(wl)
    comp_k = synth.make_comp_k(wl)
    cfg = oracle_config(wl)
    q_ref, w_ref = oracle.prepare_query(weights_np, hidden, pos, cfg)

    ck = dev(comp_k)
    q, w = retr.prepare_query(dev(hidden), dev(pos))
    results = {}
    for mode in ("max", "mean"):
        scores = retr.score(q, w, ck, None, mode)
        results[mode] = (scores, retr.keep_topk(scores, 512))
    thr_mask = retr.keep_threshold(results["max"][0], 0.5)
    dq = np.abs(host(q) - q_ref).max()

    rng = np.random.default_rng(1234)
    sb = rng.integers(0, B, 4096)
    sn = rng.integers(0, N, 4096)
    for mode in ("max", "mean"):
        s = host(results[mode][0])
        m = host(results[mode][1])
        # sampled chunks, one by one
        ref = np.empty(len(sb))
        for b in np.unique(sb):
            sel = sb == b
            k = oracle.decode_records(comp_k[b, sn[sel]])
            per = [oracle.score_layer(k, q_ref[l, b], w_ref[l, b]) for l in range(3)]
            ref[sel] = oracle.ensemble(per, mode)
        e_samp = np.abs(s[sb, sn] - ref).max()
        # full rows
        e_rows, exc = 0.0, 0
        for b in (0, B - 1):
            _, ens = oracle.score_row(comp_k[b], q_ref[:, b], w_ref[:, b], N, mode)
            e_rows = max(e_rows, max_score_err(s[b], ens))
            exc += check_topk(m[b:b + 1], s[b:b + 1], ens[None], [N], 512)
        # every row: exact top-512 of its own scores
        for b in range(B):
            own = oracle.select_topk(s[b].astype(np.float64), N, 512)
            assert np.array_equal(m[b].astype(np.uint8), own), f"row {b}"
        report(f"cfg5 full {mode} top512", max_abs_sampled=e_samp, max_abs_rows=e_rows, band_excused=exc,
               max_abs_q=dq)
        assert e_samp <= SCORE_TOL and e_rows <= SCORE_TOL
    s = host(results["max"][0])
    tm = host(thr_mask).astype(np.uint8)
    assert np.array_equal(tm, (s > 0.5).astype(np.uint8))
    _, ens0 = oracle.score_row(comp_k[0], q_ref[:, 0], w_ref[:, 0], N, "max")
    exc = check_threshold(tm[:1], s[:1], ens0[None], [N], 0.5)
    report("cfg5 full max thr0.5", band_excused=exc)
