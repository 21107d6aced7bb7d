"""fm_score_threshold, the threshold keep mask written by the score pass's
epilogue, through the C ABI.

It must give exactly what fm_score followed by fm_select_threshold gives on
the same inputs (scores bit-identical, masks identical), and so the oracle's
results within the stated tolerance and band.  Cases: workloads on row
subsets and the full-size one, ragged rows with empty and one-chunk rows,
many short rows (several rows per wave), thresholds at and around the
scores, the mean ensemble and per-layer outputs, N not a multiple of 16,
and a non-finite threshold (rejected)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from fm_cases import SCORE_TOL, check_threshold, max_score_err, oracle_scores, report, subset_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def weights_np():
    return synth.make_weights()


@pytest.fixture(scope="module")
def fm():
    import sparse_attention_chunk_amd as fm
    return fm


@pytest.fixture(scope="module")
def retr(weights_np, fm):
    r = fm.FlashMemoryRetriever(fm.weights_to_device(weights_np), max_batch=1024, max_n=1 << 18)
    yield r
    r.close()


@pytest.fixture(scope="module")
def qw(weights_np):
    """Oracle queries of 4 rows (workload 3's hidden states and positions)."""
    wl = synth.WORKLOADS[3]
    return oracle.prepare_query(weights_np, synth.make_hidden(wl)[:4], synth.make_positions(wl)[:4],
                                oracle.OracleConfig())


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def records(n, seed, rows=1):
    rng = np.random.default_rng(seed)
    return np.stack([synth.encode_records(rng.standard_normal((n, 128)).astype(np.float32)) for _ in range(rows)])


def tile_rows(q, w, B):
    """Queries of B rows cycling through the given ones."""
    idx = np.arange(B) % q.shape[1]
    return q[:, idx].astype(np.float32), w[:, idx].astype(np.float32)


def fused_vs_separate(r, q, w, comp_k, vn=None, mode="max", threshold=0.5, per_layer=False):
    """Runs both paths; asserts scores (and per-layer) bit-identical and masks
    identical; returns host scores and mask."""
    qd, wd, ck = dev(q), dev(w), dev(comp_k)
    vd = None if vn is None else dev(np.asarray(vn, np.int32))
    out = r.score_select(qd, wd, ck, vd, mode, threshold=threshold, per_layer=per_layer)
    s_f, m_f = host(out[0]), host(out[1])
    sep = r.score(qd, wd, ck, vd, mode, per_layer=per_layer)
    s_sep = sep[0] if per_layer else sep
    m_sep = r.keep_threshold(s_sep, threshold, vd)
    assert np.array_equal(s_f, host(s_sep), equal_nan=True), "fused scores differ from fm_score's"
    if per_layer:
        assert np.array_equal(host(out[2]), host(sep[1]), equal_nan=True), "fused per-layer scores differ"
    diff = m_f != host(m_sep)
    assert not diff.any(), f"fused mask differs from the separate selection in {int(diff.sum())} places"
    # Again into outputs filled with NaN scores and set mask bytes: every
    # byte and score must be written.
    from sparse_attention_chunk_amd import _lib as L
    B, N = comp_k.shape[0], comp_k.shape[1]
    s_p = torch.full((B, N), float("nan"), device="cuda")
    m_p = torch.ones((B, N), dtype=torch.bool, device="cuda")
    L.fm_score_threshold(r.ctx, qd, wd, ck, B, N, vd, L.FM_ENSEMBLE_MEAN if mode == "mean" else L.FM_ENSEMBLE_MAX,
                         float(threshold), s_p, m_p)
    assert np.array_equal(host(s_p), s_f, equal_nan=True), "scores written into NaN-filled outputs differ"
    diff = host(m_p) != m_f
    assert not diff.any(), f"mask written over set bytes differs in {int(diff.sum())} places"
    return s_f, m_f


@pytest.mark.parametrize("cid,rows,mode,threshold", [
    (1, [0], "max", 0.5),
    (2, [0, 5], "max", 0.6),
    (3, [0, 13, 31], "mean", 0.5),
    (5, [0, 29], "max", 0.5),
])
def test_workloads_against_separate_calls_and_oracle(retr, weights_np, cid, rows, mode, threshold):
    wl = synth.WORKLOADS[cid]
    hidden, pos, vn, comp_k, q_ref, w_ref = subset_inputs(wl, rows, weights_np)
    q, w = retr.prepare_query(dev(hidden), dev(pos))
    s, m = fused_vs_separate(retr, host(q), host(w), comp_k, None, mode, threshold)
    _, ens_ref = oracle_scores(comp_k, q_ref, w_ref, vn, mode)
    e = max_score_err(s, ens_ref)
    exc = check_threshold(m, s, ens_ref, vn, threshold)
    report(f"score_threshold cfg{cid} {mode} thr{threshold}", max_abs_ens=e, band_excused=exc)
    assert e <= SCORE_TOL


def test_ragged_yarn_with_empty_and_one_chunk_rows(weights_np, fm):
    wl = synth.WORKLOADS[4]
    r = fm.FlashMemoryRetriever(fm.weights_to_device(weights_np), max_batch=8, max_n=wl.n_chunks,
                                yarn={"factor": wl.yarn_factor, "orig_ctx": wl.yarn_orig_ctx,
                                      "beta_fast": wl.yarn_beta_fast, "beta_slow": wl.yarn_beta_slow})
    try:
        vn_all = synth.make_valid_n(wl)
        rows = [int(np.argmin(vn_all)), int(np.argmax(vn_all)), 7]
        hidden, pos, vn, comp_k, q_ref, w_ref = subset_inputs(wl, rows, weights_np)
        q, w = r.prepare_query(dev(hidden), dev(pos))
        vn = np.concatenate([vn, [0, 1]]).astype(np.int32)              # plus an empty and a one-chunk row
        comp_k = np.concatenate([comp_k, comp_k[:2]])
        qh, wh = host(q), host(w)
        qh = np.concatenate([qh, qh[:, :2]], axis=1)
        wh = np.concatenate([wh, wh[:, :2]], axis=1)
        s, m = fused_vs_separate(r, qh, wh, comp_k, vn, "max", 0.5)
        assert m[3].sum() == 0 and m[4, 1:].sum() == 0 and m[4, 0] == (s[4, 0] > 0.5)
        _, ens_ref = oracle_scores(comp_k[:3], q_ref, w_ref, vn[:3], "max")
        e = max_score_err(s[:3], ens_ref)
        exc = check_threshold(m[:3], s[:3], ens_ref, vn[:3], 0.5)
        report("score_threshold cfg4 ragged yarn + empty/one-chunk rows", max_abs_ens=e, band_excused=exc)
        assert e <= SCORE_TOL
    finally:
        r.close()


def test_full_size_max_and_mean(retr, weights_np):
    """B=30, N=262144, the benchmark's launch."""
    wl = synth.WORKLOADS[5]
    comp_k = synth.make_comp_k(wl)
    q, w = retr.prepare_query(dev(synth.make_hidden(wl)), dev(synth.make_positions(wl)))
    qh, wh = host(q), host(w)
    s, m = fused_vs_separate(retr, qh, wh, comp_k, None, "max", 0.5)
    assert np.array_equal(m, s > 0.5)
    fused_vs_separate(retr, qh, wh, comp_k, None, "mean", 0.5)


def test_many_short_rows(retr, qw):
    """1000 rows of 16 and fewer chunks: each wave's tiles span many rows."""
    B = 1000
    rng = np.random.default_rng(11)
    vn = rng.integers(0, 17, B).astype(np.int32)
    comp_k = records(16, 12, rows=B)
    q, w = tile_rows(*qw, B)
    for tau in (0.3, 0.5, 0.7):
        s, m = fused_vs_separate(retr, q, w, comp_k, vn, "max", tau)
        for b in range(B):
            assert not m[b, vn[b]:].any()


def test_thresholds_at_the_scores_and_ragged_tail(retr, qw):
    q, w = tile_rows(*qw, 4)
    comp_k = records(5003, 21, rows=4)          # N not a multiple of 16
    vn = np.array([5003, 4000, 17, 0], np.int32)
    s, _ = fused_vs_separate(retr, q, w, comp_k, vn, "max", 0.5)
    for tau in (float(s[0, 0]), float(s[1, 3999]), float(np.nextafter(s[0, 5], np.float32(0))), 0.0, 0.999):
        _, m = fused_vs_separate(retr, q, w, comp_k, vn, "max", tau)
        assert not m[1, 4000:].any() and not m[2, 17:].any() and not m[3].any()


def test_mean_per_layer_outputs(retr, qw):
    q, w = tile_rows(*qw, 3)
    comp_k = records(20000, 31, rows=3)
    fused_vs_separate(retr, q, w, comp_k, None, "mean", 0.55, per_layer=True)
    fused_vs_separate(retr, q, w, comp_k, None, "max", 0.6, per_layer=True)


def test_non_finite_threshold_rejected(retr, qw, fm):
    L = fm._lib
    q, w = tile_rows(*qw, 2)
    comp_k = dev(records(4096, 51, rows=2))
    qd, wd = dev(q), dev(w)
    s = torch.empty((2, 4096), device="cuda")
    m = torch.empty((2, 4096), dtype=torch.bool, device="cuda")
    for bad in (float("nan"), float("inf")):
        with pytest.raises(L.FmError) as e:
            L.fm_score_threshold(retr.ctx, qd, wd, comp_k, 2, 4096, None, L.FM_ENSEMBLE_MAX, bad, s, m)
        assert e.value.status == L.FM_EINVAL
