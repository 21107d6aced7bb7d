"""The keep-mask selection folded into the score pass (fm_score_topk +
fm_select_topk_finish, fm_score_threshold), through the C ABI.

The fused calls must give exactly what fm_score followed by fm_select_topk
or fm_select_threshold gives on the same inputs (scores bit-identical, masks
identical), and so the oracle's results within the stated tolerance and
band.  Cases: every workload on row subsets and the full-size one, ragged
rows with empty and one-chunk rows, rows beyond a score block's two
histogram slots (many short rows), K at and beyond valid_n, K = 0 and 1,
the mean ensemble and per-layer outputs, N not a multiple of 16, and rows
whose scores are all equal or largely tied (the whole-row fallback)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from fm_cases import SCORE_TOL, check_threshold, check_topk, max_score_err, oracle_scores, report, subset_inputs

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


def fused_vs_separate(r, q, w, comp_k, vn=None, mode="max", top_k=None, threshold=None, per_layer=False):
    """Runs both paths; asserts scores (and per-layer) bit-identical and masks
    identical; returns host scores and mask."""
    qd, wd, ck = dev(q), dev(w), dev(comp_k)
    vd = None if vn is None else dev(np.asarray(vn, np.int32))
    out = r.score_select(qd, wd, ck, vd, mode, top_k=top_k, threshold=threshold, per_layer=per_layer)
    s_f, m_f = host(out[0]), host(out[1])
    sep = r.score(qd, wd, ck, vd, mode, per_layer=per_layer)
    s_sep = sep[0] if per_layer else sep
    m_sep = r.keep_topk(s_sep, top_k, vd) if top_k is not None else r.keep_threshold(s_sep, threshold, vd)
    assert np.array_equal(s_f, host(s_sep), equal_nan=True), "fused scores differ from fm_score's"
    if per_layer:
        assert np.array_equal(host(out[2]), host(sep[1]), equal_nan=True), "fused per-layer scores differ"
    diff = m_f != host(m_sep)
    assert not diff.any(), f"fused mask differs from the separate selection in {int(diff.sum())} places"
    return s_f, m_f


@pytest.mark.parametrize("cid,rows,mode,top_k,threshold", [
    (1, [0], "max", 512, None),
    (2, [0, 5], "max", 512, None),
    (3, [0, 13, 31], "mean", None, 0.5),
    (3, [2, 9], "mean", 512, None),
    (5, [0, 29], "max", None, 0.5),
])
def test_workloads_against_separate_calls_and_oracle(retr, weights_np, cid, rows, mode, top_k, threshold):
    wl = synth.WORKLOADS[cid]
    hidden, pos, vn, comp_k, q_ref, w_ref = subset_inputs(wl, rows, weights_np)
    q, w = retr.prepare_query(dev(hidden), dev(pos))
    q_h, w_h = host(q), host(w)
    s, m = fused_vs_separate(retr, q_h, w_h, comp_k, None, mode, top_k, threshold)
    _, ens_ref = oracle_scores(comp_k, q_ref, w_ref, vn, mode)
    e = max_score_err(s, ens_ref)
    exc = check_topk(m, s, ens_ref, vn, top_k) if top_k is not None else check_threshold(m, s, ens_ref, vn, threshold)
    report(f"fused cfg{cid} {mode} {'top' + str(top_k) if top_k else 'thr' + str(threshold)}", max_abs_ens=e,
           band_excused=exc)
    assert e <= SCORE_TOL


def test_ragged_yarn_top1024_with_empty_and_one_chunk_rows(weights_np, fm):
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
        s, m = fused_vs_separate(r, qh, wh, comp_k, vn, "max", 1024)
        assert m[3].sum() == 0 and m[4].sum() == 1 and m[4, 0] == 1
        _, ens_ref = oracle_scores(comp_k[:3], q_ref, w_ref, vn[:3], "max")
        e = max_score_err(s[:3], ens_ref)
        exc = check_topk(m[:3], s[:3], ens_ref, vn[:3], 1024)
        report("fused cfg4 ragged yarn top1024 + empty/one-chunk rows", max_abs_ens=e, band_excused=exc)
        assert e <= SCORE_TOL
    finally:
        r.close()


def test_full_size_topk_and_threshold(retr, weights_np):
    """B=30, N=262144, the benchmark's launch: both fused modes against the
    separate calls, every row's top-512 exactly that of its own scores."""
    wl = synth.WORKLOADS[5]
    comp_k = synth.make_comp_k(wl)
    q, w = retr.prepare_query(dev(synth.make_hidden(wl)), dev(synth.make_positions(wl)))
    qh, wh = host(q), host(w)
    s, m = fused_vs_separate(retr, qh, wh, comp_k, None, "max", 512)
    for b in range(wl.batch):
        assert np.array_equal(m[b].astype(np.uint8), oracle.select_topk(s[b].astype(np.float64), wl.n_chunks, 512))
    fused_vs_separate(retr, qh, wh, comp_k, None, "mean", 512)
    _, mt = fused_vs_separate(retr, qh, wh, comp_k, None, "max", None, 0.5)
    assert np.array_equal(mt, s > 0.5)


def test_many_short_rows_beyond_two_histogram_slots(retr, qw):
    """1000 rows of 16 and fewer chunks: each score block covers several
    rows, so rows past its first two count into the global histogram."""
    B = 1000
    rng = np.random.default_rng(11)
    vn = rng.integers(0, 17, B).astype(np.int32)
    comp_k = records(16, 12, rows=B)
    q, w = tile_rows(*qw, B)
    for k in (1, 5, 16):
        s, m = fused_vs_separate(retr, q, w, comp_k, vn, "max", k)
        assert np.array_equal(m.sum(axis=1), np.minimum(vn, k))


def test_k_edges_and_ragged_tail(retr, qw):
    q, w = tile_rows(*qw, 4)
    comp_k = records(5003, 21, rows=4)          # N not a multiple of 16
    vn = np.array([5003, 4000, 17, 0], np.int32)
    for k in (0, 1, 16, 17, 4000, 5003, 6000):
        s, m = fused_vs_separate(retr, q, w, comp_k, vn, "max", k)
        assert np.array_equal(m.sum(axis=1), np.minimum(vn, k))
        assert not m[1, 4000:].any() and not m[2, 17:].any() and np.all(np.isneginf(s[1, 4000:]))


def test_mean_per_layer_outputs(retr, qw):
    q, w = tile_rows(*qw, 3)
    comp_k = records(20000, 31, rows=3)
    fused_vs_separate(retr, q, w, comp_k, None, "mean", 700, per_layer=True)
    fused_vs_separate(retr, q, w, comp_k, None, "max", 700, per_layer=True)
    fused_vs_separate(retr, q, w, comp_k, None, "mean", None, 0.55, per_layer=True)


def test_all_equal_and_largely_tied_scores(retr, qw):
    """Zero records score exactly 1/2: a row of them puts every chunk in one
    histogram bin (whole-row fallback, ties to the lowest indices); a row
    with a zero-record majority ties across the K-th score."""
    q, w = tile_rows(*qw, 3)
    N = 30000
    comp_k = records(N, 41, rows=3)
    comp_k[0] = 0                                 # every score 0.5
    tied = np.random.default_rng(42).random(N) < 0.7
    comp_k[1, tied] = 0                           # 70% of the chunks at 0.5
    comp_k[2, :N // 2] = comp_k[2, N // 2:]       # duplicated records: pairs of equal scores
    for k in (1, 512, 9000, 25000):
        s, m = fused_vs_separate(retr, q, w, comp_k, None, "max", k)
        assert np.all(s[0] == 0.5)
        assert m[0, :k].all() and not m[0, k:].any()


def test_finish_must_follow_a_matching_score_topk(retr, qw, fm):
    L = fm._lib
    q, w = tile_rows(*qw, 2)
    comp_k = dev(records(4096, 51, rows=2))
    qd, wd = dev(q), dev(w)
    s = torch.empty((2, 4096), device="cuda")
    m = torch.empty((2, 4096), dtype=torch.bool, device="cuda")
    L.fm_score_topk(retr.ctx, qd, wd, comp_k, 2, 4096, None, L.FM_ENSEMBLE_MAX, 64, s, m)
    with pytest.raises(L.FmError) as e:
        L.fm_select_topk_finish(retr.ctx, s, 2, 4096, None, 65, m)
    assert e.value.status == L.FM_EINVAL
    other = torch.empty_like(m)
    with pytest.raises(L.FmError):
        L.fm_select_topk_finish(retr.ctx, s, 2, 4096, None, 64, other)
    L.fm_select_topk_finish(retr.ctx, s, 2, 4096, None, 64, m)
    torch.cuda.synchronize()
    assert int(m.sum()) == 128
    with pytest.raises(L.FmError):
        L.fm_score_threshold(retr.ctx, qd, wd, comp_k, 2, 4096, None, L.FM_ENSEMBLE_MAX, float("nan"), s, m)
