"""The largest batch the C ABI accepts: B = max_batch = 4096 rows.

Query preparation for 4096 rows (128 groups of 32 rows in the projections)
is compared with the oracle on sampled rows, the first and last of row
groups among them.  The score pass over 4096 ragged rows of 48 chunks
(every row length from empty to whole, valid_n below 0 and above N; the
ragged plan's block then takes four consecutive rows per thread) starts
from seeded synthetic queries of the prepared ones' size (q ~ N(0, 1), w ~
N(0, 0.011)), so no oracle input comes from the GPU: every score against
the oracle, the top-K mask exactly the top-K of the GPU's own scores and
the oracle's outside the band, and likewise the threshold mask written by
the score pass.  Records past a row's valid_n are 0xFF (NaN codes and
scale): never read."""

import numpy as np
import pytest
import torch

import oracle
import synth
from fm_cases import Q_TOL, SCORE_TOL, W_TOL, check_threshold, check_topk, max_score_err, oracle_scores, report

pytestmark = pytest.mark.gpu

B = 4096
N = 48


@pytest.fixture(scope="module")
def weights_np():
    return synth.make_weights()


@pytest.fixture(scope="module")
def retr(weights_np):
    import sparse_attention_chunk_amd as fm
    r = fm.FlashMemoryRetriever(fm.weights_to_device(weights_np), max_batch=B, max_n=N)
    yield r
    r.close()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def test_prepare_query_at_max_batch(retr, weights_np):
    rng = np.random.default_rng(4096)
    hidden = rng.standard_normal((B, 4096)).astype(np.float32)
    pos = rng.integers(0, 1 << 20, B).astype(np.int64)
    q, w = retr.prepare_query(dev(hidden), dev(pos))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 31, 32, 33, 2047, 2048, 4063, 4064, 4095], rng.integers(0, B, 6)]))
    q_ref, w_ref = oracle.prepare_query(weights_np, hidden[rows], pos[rows], oracle.OracleConfig())
    it = torch.from_numpy(rows).cuda()
    eq = float(np.abs(q.index_select(1, it).cpu().numpy() - q_ref).max())
    ew = float(np.abs(w.index_select(1, it).cpu().numpy() - w_ref).max())
    report(f"prepare B = {B}, {len(rows)} sampled rows", max_abs_q=eq, max_abs_w=ew)
    assert eq <= Q_TOL and ew <= W_TOL


@pytest.fixture(scope="module")
def ragged_inputs():
    rng = np.random.default_rng(4097)
    q = rng.standard_normal((3, B, 64, 128)).astype(np.float32)
    w = (rng.standard_normal((3, B, 64)) * 0.011).astype(np.float32)
    vn = rng.integers(-3, N + 6, B).astype(np.int32)
    vn[:8] = [0, N, -1, N + 7, 1, 16, 17, N - 1]
    vn[-1] = N
    ck = synth.encode_records(rng.standard_normal((B * N, 128)).astype(np.float32)).reshape(B, N, 132)
    vc = np.clip(vn, 0, N)
    for b in range(B):
        ck[b, vc[b]:] = 0xFF
    return q, w, vn, vc, ck


@pytest.mark.parametrize("mode", ["max", "mean"])
def test_ragged_rows_at_max_batch(retr, ragged_inputs, mode):
    q, w, vn, vc, ck = ragged_inputs
    qd, wd, ckd, vd = dev(q), dev(w), dev(ck), dev(vn)
    s, p = retr.score(qd, wd, ckd, vd, mode, per_layer=True)
    torch.cuda.synchronize()
    per_ref, ens_ref = oracle_scores(ck, q.astype(np.float64), w.astype(np.float64), vc, mode)
    s_h, p_h = s.cpu().numpy(), p.cpu().numpy()
    e = max(max_score_err(s_h, ens_ref), max_score_err(p_h, per_ref))
    if mode == "max":
        m = retr.keep_topk(s, 5, vd)
        exc = check_topk(m.cpu().numpy(), s_h, ens_ref, vc, 5)
    else:
        s2, m = retr.score_select(qd, wd, ckd, vd, mode, threshold=0.5)
        assert torch.equal(s2, s)
        exc = check_threshold(m.cpu().numpy(), s_h, ens_ref, vc, 0.5)
    report(f"B = {B} ragged rows of {N}, {mode}", max_abs=e, band_excused=exc)
    assert e <= SCORE_TOL
