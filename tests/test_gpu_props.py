"""GPU properties and edge cases through the C ABI: determinism, chunk
permutation, row independence, ties, zero and negative-scale records,
records at the ends of the format (saturating scores), tiny and large
(f16-exact) query magnitudes, ragged and degenerate sizes, and the
selection kernels on constructed scores (compared exactly with the oracle's
selection of the same scores)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from fm_cases import SCORE_TOL, max_score_err, oracle_scores, report

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def weights_np():
    return synth.make_weights()


@pytest.fixture(scope="module")
def retr(weights_np):
    import sparse_attention_chunk_amd as fm
    r = fm.FlashMemoryRetriever(fm.weights_to_device(weights_np), max_batch=64, max_n=1 << 17)
    yield r
    r.close()


@pytest.fixture(scope="module")
def qw(weights_np):
    """Oracle queries of 4 rows (cfg 3 hidden states, random positions)."""
    wl = synth.WORKLOADS[3]
    hidden = synth.make_hidden(wl)[:4]
    pos = synth.make_positions(wl)[:4]
    q, w = oracle.prepare_query(weights_np, hidden, pos, oracle.OracleConfig())
    return q, w


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def records(n, seed, rows=1):
    rng = np.random.default_rng(seed)
    return np.stack([synth.encode_records(rng.standard_normal((n, 128)).astype(np.float32)) for _ in range(rows)])


def run(retr, q, w, comp_k, vn=None, mode="max"):
    qd, wd = dev(q.astype(np.float32)), dev(w.astype(np.float32))
    s, p = retr.score(qd, wd, dev(comp_k), None if vn is None else dev(np.asarray(vn, np.int32)), mode,
                      per_layer=True)
    return host(s), host(p)


def test_bit_identical_run_to_run(retr, qw):
    q, w = qw
    ck = records(5000, 1, rows=2)
    a, pa = run(retr, q[:, :2], w[:, :2], ck)
    b, pb = run(retr, q[:, :2], w[:, :2], ck)
    assert np.array_equal(a, b) and np.array_equal(pa, pb)


def test_chunk_permutation_permutes_scores(retr, qw):
    q, w = qw
    ck = records(3000, 2)
    perm = np.random.default_rng(3).permutation(3000)
    a, _ = run(retr, q[:, :1], w[:, :1], ck)
    b, _ = run(retr, q[:, :1], w[:, :1], ck[:, perm])
    assert np.array_equal(a[0, perm], b[0])


def test_row_independence(retr, qw):
    q, w = qw
    ck = records(2048, 4, rows=3)
    a, _ = run(retr, q[:, :3], w[:, :3], ck)
    b, _ = run(retr, q[:, 1:2], w[:, 1:2], ck[1:2])
    assert np.array_equal(a[1], b[0])


@pytest.mark.parametrize("n", [1, 15, 16, 17, 4095, 4097, 5000])
def test_ragged_sizes_match_oracle(retr, qw, n):
    q, w = qw
    ck = records(n, 10 + n, rows=2)
    vn = [n, max(0, n // 3)]
    ck[1, vn[1]:] = 0xFF                      # tail must not be read
    s, p = run(retr, q[:, :2], w[:, :2], ck, vn)
    per_ref, ens_ref = oracle_scores(ck, q[:, :2], w[:, :2], vn, "max")
    e = max(max_score_err(s, ens_ref), max_score_err(p, per_ref))
    report(f"ragged n={n}", max_abs=e)
    assert e <= SCORE_TOL


def test_many_ragged_rows_share_waves(retr, qw):
    """40 rows of assorted valid lengths (empty, sub-tile, one tile plus one,
    full): the valid tiles of all rows are split evenly over the waves, so
    waves start and end inside rows and step over empty ones."""
    q, w = qw
    B, n = 40, 3000
    pick = [i % 4 for i in range(B)]
    qb, wb = q[:, pick], w[:, pick]
    vn = np.array([0, 1, 15, 16, 17, 100, 2999, 3000, 0, 0] * 4, np.int32)
    vn[10:20] = np.random.default_rng(31).integers(0, n + 1, 10)
    ck = records(n, 30, rows=B)
    for b in range(B):
        ck[b, vn[b]:] = 0xFF
    for mode in ("max", "mean"):
        s, p = run(retr, qb, wb, ck, vn, mode)
        per_ref, ens_ref = oracle_scores(ck, qb, wb, vn, mode)
        e = max(max_score_err(s, ens_ref), max_score_err(p, per_ref))
        report(f"40 ragged rows {mode}", max_abs=e)
        assert e <= SCORE_TOL


def test_empty_rows_and_zero_valid(retr, qw, fm_lib):
    q, w = qw
    ck = records(64, 5, rows=2)
    s, p = run(retr, q[:, :2], w[:, :2], ck, [0, 64])
    assert np.all(np.isneginf(s[0])) and np.all(np.isneginf(p[:, 0]))
    mask = retr.keep_topk(dev(s), 10, dev(np.array([0, 64], np.int32)))
    m = host(mask)
    assert m[0].sum() == 0 and m[1].sum() == 10
    # B == 0 and N == 0 are empty problems: FM_OK, nothing written
    assert fm_lib.LIB.fm_score(retr.ctx, 0, 0, 0, 0, 5, None, 0, 0, None, None) == 0
    assert fm_lib.LIB.fm_select_topk(retr.ctx, 0, 3, 0, None, 5, 0, None) == 0


@pytest.fixture(scope="module")
def fm_lib():
    from sparse_attention_chunk_amd import _lib
    return _lib


def test_zero_records_score_exactly_half(retr, qw):
    q, w = qw
    ck = np.zeros((1, 100, 132), np.uint8)     # codes 0, scale 0
    s, p = run(retr, q[:, :1], w[:, :1], ck)
    assert np.all(s == 0.5) and np.all(p == 0.5)


def test_negative_and_mixed_scales(retr, qw):
    q, w = qw
    ck = records(1000, 6)
    sc = ck[0, :, 128:].copy().view("<f4")[:, 0]
    sc[::3] *= -1.0                            # every third chunk: negative scale
    ck[0, :, 128:] = sc.astype("<f4").view(np.uint8).reshape(-1, 4)
    s, p = run(retr, q[:, :1], w[:, :1], ck)
    per_ref, ens_ref = oracle_scores(ck, q[:, :1], w[:, :1], [1000], "max")
    e = max(max_score_err(s, ens_ref), max_score_err(p, per_ref))
    report("negative scales", max_abs=e)
    assert e <= SCORE_TOL


@pytest.mark.parametrize("fp8", [False, True])
def test_tiny_queries(retr, qw, fp8):
    """Queries scaled by 2^-20: most f16 query entries fall in the subnormal
    range and the linear term's block scale is far from 1.  Scores stay
    within the tolerance of the oracle's on the same queries (near 1/2,
    with nothing flushed to NaN or infinity)."""
    q, w = qw
    qs = q[:, :2] * 2.0 ** -20
    ck = records(3000, 11, rows=2)
    s, p = retr.score(dev(qs.astype(np.float32)), dev(w[:, :2].astype(np.float32)), dev(ck), None, "max",
                      per_layer=True, fp8=fp8)
    per_ref, ens_ref = oracle_scores(ck, qs, w[:, :2], [3000, 3000], "max")
    e = max(max_score_err(host(s), ens_ref), max_score_err(host(p), per_ref))
    report(f"q x 2^-20 ({'fp8' if fp8 else 'f16'})", max_abs=e)
    assert e <= SCORE_TOL


def test_large_f16_exact_queries(retr, qw):
    """Queries 256 times their usual size (most sigmoids saturate) but exactly
    representable in f16, so the kernel's one rounding of q is exact and
    what remains (the exact decode, fp32 products and sums, the linear term's
    three e4m3 parts, the sigmoid) must stay within the tolerance of the
    oracle on the same queries.  (With unrepresentable queries at this size,
    the rounding of q to f16 alone moves scores by up to about 2.4e-2: the
    score error of the f16 path grows with the size of the logits, and the
    2e-3 bound holds at the prepared queries' size.)"""
    q, w = qw
    qs = q[:, :2].astype(np.float16).astype(np.float64) * 2.0 ** 8
    ck = records(3000, 12, rows=2)
    s, p = retr.score(dev(qs.astype(np.float32)), dev(w[:, :2].astype(np.float32)), dev(ck), None, "max",
                      per_layer=True)
    per_ref, ens_ref = oracle_scores(ck, qs, w[:, :2], [3000, 3000], "max")
    e = max(max_score_err(host(s), ens_ref), max_score_err(host(p), per_ref))
    report("q x 2^8, f16-exact", max_abs=e)
    assert e <= SCORE_TOL


@pytest.mark.parametrize("fp8", [False, True])
def test_extreme_codes_and_saturating_scales(retr, qw, fp8):
    """Records at the ends of the format: every code +-448 (the largest
    e4m3fn magnitude) or the smallest subnormal (2^-9), and scales from
    1e-30 up to 3e38, where |s| times a logit overflows to +-inf and the
    sigmoid must give exactly 0 or 1 (never NaN).  Scores against the oracle;
    the top-K among the many exact ties at 0 and 1 goes to the lowest
    indices."""
    q, w = qw
    rng = np.random.default_rng(31)
    n = 16 * 40
    ck = records(n, 32)[0]
    kinds = rng.integers(0, 6, n)
    for c in range(n):
        kind = kinds[c]
        if kind == 0:
            ck[c, :128] = 0x7E                                       # +448
        elif kind == 1:
            ck[c, :128] = 0xFE                                       # -448
        elif kind == 2:
            ck[c, :128] = np.where(rng.integers(0, 2, 128) == 1, 0x01, 0x81)   # +-2^-9
        scale = [1.0, 1.0, 1e-30, 1e36, -3e38, 1e30][kind] * (1 + rng.uniform())
        ck[c, 128:] = np.frombuffer(np.float32(min(scale, 3.4e38) if scale > 0 else max(scale, -3.4e38)).tobytes(),
                                    np.uint8)
    ck = ck[None]
    qs, ws = q[:, :1], w[:, :1]
    s, p = retr.score(dev(qs.astype(np.float32)), dev(ws.astype(np.float32)), dev(ck), None, "max",
                      per_layer=True, fp8=fp8)
    s_h, p_h = host(s), host(p)
    assert np.all(np.isfinite(s_h)) and np.all(np.isfinite(p_h))
    per_ref, ens_ref = oracle_scores(ck, qs, ws, [n], "max")
    e = max(max_score_err(s_h, ens_ref), max_score_err(p_h, per_ref))
    sat = int(np.sum((s_h == 0.0) | (s_h == 1.0)))
    report(f"extreme codes and scales ({'fp8' if fp8 else 'f16'})", max_abs=e, saturated=sat)
    assert e <= SCORE_TOL
    for k in (7, 200):
        m = host(retr.keep_topk(s, k))
        assert np.array_equal(m[0].astype(np.uint8), oracle.select_topk(s_h[0].astype(np.float64), n, k))


def test_identical_records_tie_to_lowest_index(retr, qw):
    q, w = qw
    one = records(1, 7)[0, 0]
    ck = np.tile(one, (1, 300, 1))
    s, _ = run(retr, q[:, :1], w[:, :1], ck)
    assert np.all(s[0] == s[0, 0])
    m = host(retr.keep_topk(dev(s), 37))
    assert list(np.nonzero(m[0])[0]) == list(range(37))


# --------------------------------------------------------------------------- selection on constructed scores

@pytest.mark.parametrize("n,k", [(1, 1), (10, 3), (4096, 512), (4097, 4096), (70000, 1024), (131072, 512)])
def test_topk_many_ties_exact(retr, n, k):
    rng = np.random.default_rng(n + k)
    s = np.round(rng.uniform(0, 1, (3, n)), 3).astype(np.float32)   # heavy ties
    vn = np.array([n, max(1, n // 2), 0], np.int32)
    m = host(retr.keep_topk(dev(s), k, dev(vn)))
    for b in range(3):
        assert np.array_equal(m[b].astype(np.uint8), oracle.select_topk(s[b].astype(np.float64), int(vn[b]), k))


def test_topk_all_equal_and_degenerate_k(retr):
    s = np.full((2, 9000), 0.25, np.float32)
    m = host(retr.keep_topk(dev(s), 4500))
    assert all(list(np.nonzero(m[b])[0]) == list(range(4500)) for b in range(2))
    assert host(retr.keep_topk(dev(s), 0)).sum() == 0
    assert host(retr.keep_topk(dev(s), 9000)).all()
    assert host(retr.keep_topk(dev(s), 100000)).all()


def test_topk_with_negative_inf_and_signed_values(retr):
    rng = np.random.default_rng(11)
    s = rng.standard_normal((2, 5000)).astype(np.float32)
    s[0, ::7] = -np.inf
    s[1, :10] = 0.0
    s[1, 10:20] = -0.0
    for k in (1, 100, 4000, 4999):
        m = host(retr.keep_topk(dev(s), k))
        for b in range(2):
            assert np.array_equal(m[b].astype(np.uint8), oracle.select_topk(s[b].astype(np.float64), 5000, k)), (b, k)


@pytest.mark.parametrize("tau", [0.5, 0.0, 0.9])
def test_threshold_strict_exact(retr, tau):
    rng = np.random.default_rng(12)
    s = np.round(rng.uniform(0, 1, (4, 10001)), 2).astype(np.float32)
    s[0, :50] = np.float32(tau)
    vn = np.array([10001, 5000, 0, 1], np.int32)
    m = host(retr.keep_threshold(dev(s), tau, dev(vn)))
    for b in range(4):
        assert np.array_equal(m[b].astype(np.uint8), oracle.select_threshold(s[b].astype(np.float64), int(vn[b]), tau))


def test_topk_top_scores_packed_in_few_tiles(retr):
    """The top scores fill runs of consecutive 16-chunk tiles, so the K-th
    largest tile maximum lies far below the K-th score: most of the row's
    candidates come from low tiles, and the finish may overflow LDS and
    select over the whole row.  The result is still the exact top-K."""
    n, k, run = 65536, 512, 64
    rng = np.random.default_rng(21)
    s = rng.uniform(0.05, 0.2, (2, n)).astype(np.float32)
    starts = [r * (n - run) // 63 for r in range(64)]
    vals = np.linspace(0.9, 0.99, 64 * run).astype(np.float32)
    i = 0
    for st in starts:
        s[0, st:st + run] = vals[i:i + run]
        i += run
    s[1] = s[0][::-1]                       # second row: a different layout, same values
    for kk in (k, 4096, 5000):
        m = host(retr.keep_topk(dev(s), kk))
        for b in range(2):
            assert np.array_equal(m[b].astype(np.uint8), oracle.select_topk(s[b].astype(np.float64), n, kk)), (b, kk)


def test_topk_many_candidates_in_the_last_bin(retr):
    """3000 scattered chunks within one histogram bin (1/2048 wide) above a
    low background, K = 1500: the candidates fit in LDS but more than 1024 of
    them share the K-th score's bin, which is then split by radix passes."""
    n = 65536
    rng = np.random.default_rng(23)
    s = rng.uniform(0.0, 0.5, (2, n)).astype(np.float32)
    pos = rng.choice(n, 3000, replace=False)
    s[0, pos] = (0.9 + rng.integers(0, 400, 3000) * 1e-7).astype(np.float32)   # ties too
    s[1, pos] = np.float32(0.9)                                                # all equal
    for k in (1, 1500, 2999, 3000, 3001):
        m = host(retr.keep_topk(dev(s), k))
        for b in range(2):
            assert np.array_equal(m[b].astype(np.uint8), oracle.select_topk(s[b].astype(np.float64), n, k)), (b, k)


def test_topk_many_short_rows(retr):
    """64 rows of at most 40 chunks (one to three tiles), every K edge."""
    rng = np.random.default_rng(24)
    B, n = 64, 40
    s = np.round(rng.uniform(0, 1, (B, n)), 2).astype(np.float32)
    vn = rng.integers(0, n + 1, B).astype(np.int32)
    for k in (0, 1, 2, 15, 16, 17, 39, 40):
        m = host(retr.keep_topk(dev(s), k, dev(vn)))
        for b in range(B):
            assert np.array_equal(m[b].astype(np.uint8), oracle.select_topk(s[b].astype(np.float64), int(vn[b]), k))


def test_topk_rows_beyond_the_register_tiles(weights_np):
    """Rows of more than 16384 tiles (N > 262144): the tile maxima beyond the
    registers are read again for the histogram and the compaction."""
    import sparse_attention_chunk_amd as fm
    r = fm.FlashMemoryRetriever(fm.weights_to_device(weights_np), max_batch=2, max_n=600000)
    try:
        rng = np.random.default_rng(25)
        n = 600000
        s = rng.uniform(0, 1, (2, n)).astype(np.float32)
        s[1, 590000:] += 0.5                     # the top of row 1 sits past the register tiles
        vn = np.array([n, 599999], np.int32)
        for k in (512, 2048):
            m = host(r.keep_topk(dev(s), k, dev(vn)))
            for b in range(2):
                assert np.array_equal(m[b].astype(np.uint8),
                                      oracle.select_topk(s[b].astype(np.float64), int(vn[b]), k)), (b, k)
    finally:
        r.close()


@pytest.mark.parametrize("n,k", [(5003, 17), (77, 5), (40000, 512), (3, 1), (8192, 512), (8193, 512)])
def test_topk_and_threshold_write_every_byte(retr, n, k):
    """Masks filled with ones beforehand: every byte of the [B][N] mask is
    written (N odd, ragged rows, rows kept whole and empty), on both sides of
    the row length (8192) up to which top-K takes one launch per row."""
    from sparse_attention_chunk_amd import _lib as L
    rng = np.random.default_rng(n)
    B = 5
    s = rng.uniform(0, 1, (B, n)).astype(np.float32)
    vn = np.array([n, n - 1, min(k, n), 0, max(1, n // 3)], np.int32)
    sd, vd = dev(s), dev(vn)
    m = torch.ones((B, n), dtype=torch.bool, device="cuda")
    L.fm_select_topk(retr.ctx, sd, B, n, vd, k, m)
    mt = torch.ones((B, n), dtype=torch.bool, device="cuda")
    L.fm_select_threshold(retr.ctx, sd, B, n, vd, 0.5, mt)
    m, mt = host(m), host(mt)
    for b in range(B):
        assert np.array_equal(m[b].astype(np.uint8), oracle.select_topk(s[b].astype(np.float64), int(vn[b]), k)), b
        assert np.array_equal(mt[b].astype(np.uint8), oracle.select_threshold(s[b].astype(np.float64), int(vn[b]),
                                                                                0.5)), b


def test_topk_large_candidate_lists(retr):
    """All-equal rows longer than the LDS staging: every chunk is a candidate."""
    n = 100000
    s = np.full((2, n), 0.5, np.float32)
    s[1, ::3] = 0.25
    for k in (5000, 30000):
        m = host(retr.keep_topk(dev(s), k))
        for b in range(2):
            assert np.array_equal(m[b].astype(np.uint8), oracle.select_topk(s[b].astype(np.float64), n, k)), (b, k)
