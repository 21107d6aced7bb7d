"""fm_score_fp8 (the fp8-MFMA score) against the fp64 oracle, through the C
ABI: the same 2e-3 score bound and mask checks as fm_score on every
workload, plus the cases its query split meets (zero heads, zero weights,
heads of very different magnitude, ragged tile tails)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from fm_cases import (SCORE_TOL, check_threshold, check_topk, max_score_err, oracle_config, oracle_scores, report,
                      subset_inputs, yarn_kwargs)

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


def score_fp8(r, q, w, comp_k, vn=None, mode="max"):
    return r.score(q, w, comp_k, vn, mode, per_layer=True, fp8=True)


@pytest.mark.parametrize("mode", ["max", "mean"])
def test_fp8_score_from_oracle_queries(retr, weights_np, mode):
    wl = synth.WORKLOADS[1]
    _, _, vn, comp_k, q, w = subset_inputs(wl, [0], weights_np)
    per_ref, ens_ref = oracle_scores(comp_k, q, w, vn, mode)
    s, p = score_fp8(retr, dev(q.astype(np.float32)), dev(w.astype(np.float32)), dev(comp_k), None, mode)
    e1, e2 = max_score_err(host(s), ens_ref), max_score_err(host(p), per_ref)
    report(f"fp8 score cfg1 {mode} (oracle q)", max_abs_ens=e1, max_abs_per_layer=e2)
    assert e1 <= SCORE_TOL and e2 <= SCORE_TOL


def _whole_pass(r, wl, rows, weights_np, mode, top_k, threshold, use_valid=False):
    hidden, pos, vn, comp_k, q_ref, w_ref = subset_inputs(wl, rows, weights_np)
    per_ref, ens_ref = oracle_scores(comp_k, q_ref, w_ref, vn, mode)
    q, w = r.prepare_query(dev(hidden), dev(pos))
    vdev = dev(vn.astype(np.int32)) if use_valid else None
    scores, per = score_fp8(r, q, w, dev(comp_k), vdev, mode)
    mask = r.keep_topk(scores, top_k, vdev) if top_k is not None else r.keep_threshold(scores, threshold, vdev)
    s, p, m = host(scores), host(per), host(mask)
    e_ens, e_per = max_score_err(s, ens_ref), max_score_err(p, per_ref)
    if top_k is not None:
        exc = check_topk(m, s, ens_ref, vn, top_k)
    else:
        exc = check_threshold(m, s, ens_ref, vn, threshold)
    return e_ens, e_per, exc


@pytest.mark.parametrize("cid,rows,mode,top_k,thr", [
    (1, [0], "max", 512, None),
    (2, [0, 5], "max", 512, None),
    (3, [0, 13, 31], "mean", None, 0.5),
])
def test_fp8_whole_pass(retr, weights_np, cid, rows, mode, top_k, thr):
    e_ens, e_per, exc = _whole_pass(retr, synth.WORKLOADS[cid], rows, weights_np, mode, top_k, thr)
    report(f"fp8 cfg{cid} rows {rows} {mode}", max_abs_ens=e_ens, max_abs_per_layer=e_per, band_excused=exc)
    assert e_ens <= SCORE_TOL and e_per <= SCORE_TOL


def test_fp8_ragged_yarn_top1024(retr_yarn, weights_np):
    wl = synth.WORKLOADS[4]
    vn_all = synth.make_valid_n(wl)
    rows = sorted({int(np.argmin(vn_all)), int(np.argmax(vn_all)), 7, 30})
    e_ens, e_per, exc = _whole_pass(retr_yarn, wl, rows, weights_np, "max", 1024, None, use_valid=True)
    report("fp8 cfg4 ragged yarn max top1024", max_abs_ens=e_ens, max_abs_per_layer=e_per, band_excused=exc)
    assert e_ens <= SCORE_TOL and e_per <= SCORE_TOL


def test_fp8_query_split_edge_cases(retr, weights_np):
    """Heads of zero, tiny and huge magnitude in one row (each head has its
    own power-of-two scale), a layer with all-zero weights (zero linear
    term) and one with a zero query; N = 1, 17 and 4099 (ragged tails)."""
    wl = synth.WORKLOADS[1]
    _, _, _, comp_k, q, w = subset_inputs(wl, [0], weights_np)
    q = q.copy()
    w = w.copy()
    q[0, 0, 3] = 0.0                 # one zero head
    q[0, 0, 5] *= 1e-12              # tiny head
    q[0, 0, 9] *= 1e6                # huge head
    q[0, 0, 10] *= 37.0
    w[0, 0, 9] *= 1e-6               # keeps the huge head's logit moderate
    w[1, 0, :] = 0.0                 # layer 1: zero weights -> zero linear term, sigmoid(0)
    q[2, 0, :, :] = 0.0              # layer 2: zero query
    for n in (1, 17, 4099):
        ck = comp_k[:, :n]
        vn = np.array([n])
        per_ref, ens_ref = oracle_scores(ck, q, w, vn, "max")
        s, p = score_fp8(retr, dev(q.astype(np.float32)), dev(w.astype(np.float32)), dev(ck))
        e1, e2 = max_score_err(host(s), ens_ref), max_score_err(host(p), per_ref)
        report(f"fp8 edge heads n={n}", max_abs_ens=e1, max_abs_per_layer=e2)
        assert e1 <= SCORE_TOL and e2 <= SCORE_TOL
        assert np.all(host(p)[1:] == 0.5)  # layers 1 and 2 score sigmoid(0) exactly


def test_fp8_full_size_sampled(retr, weights_np):
    """B=30, N=262144 (the benchmark's launch): sampled chunks one by one and
    a full row against the oracle, every row's top-512 exactly that of its
    own scores, and the fp8 scores within 2e-3 of the f16 ones everywhere."""
    wl = synth.WORKLOADS[5]
    B, N = wl.batch, wl.n_chunks
    hidden = synth.make_hidden(wl)
    pos = synth.make_positions(wl)
    comp_k = synth.make_comp_k(wl)
    q_ref, w_ref = oracle.prepare_query(weights_np, hidden, pos, oracle_config(wl))
    ck = dev(comp_k)
    q, w = retr.prepare_query(dev(hidden), dev(pos))
    s8 = retr.score(q, w, ck, None, "max", fp8=True)
    m8 = retr.keep_topk(s8, 512)
    s16 = retr.score(q, w, ck, None, "max")
    s, m, s_f16 = host(s8), host(m8), host(s16)
    rng = np.random.default_rng(4321)
    sb, sn = rng.integers(0, B, 4096), rng.integers(0, N, 4096)
    ref = np.empty(len(sb))
    for b in np.unique(sb):
        sel = sb == b
        k = oracle.decode_records(comp_k[b, sn[sel]])
        ref[sel] = oracle.ensemble([oracle.score_layer(k, q_ref[l, b], w_ref[l, b]) for l in range(3)], "max")
    e_samp = np.abs(s[sb, sn] - ref).max()
    _, ens = oracle.score_row(comp_k[B - 1], q_ref[:, B - 1], w_ref[:, B - 1], N, "max")
    e_row = max_score_err(s[B - 1], ens)
    exc = check_topk(m[B - 1:], s[B - 1:], ens[None], [N], 512)
    for b in range(B):
        own = oracle.select_topk(s[b].astype(np.float64), N, 512)
        assert np.array_equal(m[b].astype(np.uint8), own), f"row {b}"
    d16 = float(np.abs(s - s_f16).max())
    report("fp8 cfg5 full max top512", max_abs_sampled=e_samp, max_abs_row=e_row, band_excused=exc,
           max_abs_vs_f16=d16)
    assert e_samp <= SCORE_TOL and e_row <= SCORE_TOL and d16 <= SCORE_TOL


def test_fp8_argument_errors(retr):
    from sparse_attention_chunk_amd import _lib
    L = _lib.LIB
    q = torch.zeros((3, 1, 64, 128), device="cuda")
    w = torch.zeros((3, 1, 64), device="cuda")
    ck = torch.zeros((1, 16, 132), dtype=torch.uint8, device="cuda")
    s = torch.zeros((1, 16), device="cuda")
    assert L.fm_score_fp8(retr.ctx, q.data_ptr(), w.data_ptr(), ck.data_ptr(), 1, 16, None, 7, s.data_ptr(), None,
                          None) == _lib.FM_EINVAL
    assert L.fm_score_fp8(retr.ctx, q.data_ptr() + 4, w.data_ptr(), ck.data_ptr(), 1, 16, None, 0, s.data_ptr(),
                          None, None) == _lib.FM_EINVAL
    assert L.fm_score_fp8(retr.ctx, q.data_ptr(), w.data_ptr(), ck.data_ptr(), 65, 16, None, 0, s.data_ptr(), None,
                          None) == _lib.FM_EINVAL
    assert L.fm_score_fp8(retr.ctx, None, None, None, 0, 0, None, 0, None, None, None) == _lib.FM_OK


# --------------------------------------------------------------------------- properties of the fp8 path

def _records(n, seed, rows=1):
    rng = np.random.default_rng(seed)
    return np.stack([synth.encode_records(rng.standard_normal((n, 128)).astype(np.float32)) for _ in range(rows)])


@pytest.fixture(scope="module")
def qw4(weights_np):
    wl = synth.WORKLOADS[3]
    return oracle.prepare_query(weights_np, synth.make_hidden(wl)[:4], synth.make_positions(wl)[:4],
                                oracle.OracleConfig())


def _run8(retr, q, w, ck):
    s, p = score_fp8(retr, dev(q.astype(np.float32)), dev(w.astype(np.float32)), dev(ck))
    return host(s), host(p)


def test_fp8_bit_identical_and_row_independent(retr, qw4):
    q, w = qw4
    ck = _records(5000, 11, rows=3)
    a, pa = _run8(retr, q[:, :3], w[:, :3], ck)
    b, pb = _run8(retr, q[:, :3], w[:, :3], ck)
    assert np.array_equal(a, b) and np.array_equal(pa, pb)
    c, _ = _run8(retr, q[:, 1:2], w[:, 1:2], ck[1:2])
    assert np.array_equal(a[1], c[0])


def test_fp8_zero_records_and_negative_scales(retr, qw4):
    q, w = qw4
    s, p = _run8(retr, q[:, :1], w[:, :1], np.zeros((1, 100, 132), np.uint8))
    assert np.all(s == 0.5) and np.all(p == 0.5)
    ck = _records(1000, 12)
    sc = ck[0, :, 128:].copy().view("<f4")[:, 0]
    sc[::3] *= -1.0
    ck[0, :, 128:] = sc.astype("<f4").view(np.uint8).reshape(-1, 4)
    s, p = _run8(retr, q[:, :1], w[:, :1], ck)
    per_ref, ens_ref = oracle_scores(ck, q[:, :1], w[:, :1], [1000], "max")
    e = max(max_score_err(s, ens_ref), max_score_err(p, per_ref))
    report("fp8 negative scales", max_abs=e)
    assert e <= SCORE_TOL
