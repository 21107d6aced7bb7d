"""The longest row the C ABI accepts: B = 1, N = 2^26 chunks (8.9 GB of
records in one row).  Record byte offsets pass 2^32 inside the row, every
wave's share of the tile list is 4096 tiles, and the top-K scan covers 2^22
tiles of 16 chunks.

Records are drawn on the GPU (torch's generator, seeded): code bytes with
the top exponent bit cleared (|value| <= 1.875, never the NaN code) and a
random sign, scales of either sign with magnitude in [0.02, 0.2).  Scores
(f16 and fp8 paths, ensemble and per layer) are compared with the oracle on
sampled chunks: the first and last ones, those on both sides of the 2^32-byte
record offset and of wave-share edges, and random ones.  The top-K and
threshold masks are compared exactly with the oracle's selection of the
GPU's own scores over the whole row, and so are the next rows' passes at
this length: the resident set and recall delta between two masks, and the
top-K within a resident list."""

import numpy as np
import pytest
import torch

import oracle
import synth
from fm_cases import SCORE_TOL, max_score_err, report

pytestmark = pytest.mark.gpu

N = 1 << 26
RECORD = 132


@pytest.fixture(scope="module")
def big():
    import sparse_attention_chunk_amd as fm
    weights_np = synth.make_weights()
    r = fm.FlashMemoryRetriever(fm.weights_to_device(weights_np), max_batch=1, max_n=N)
    wl = synth.WORKLOADS[3]
    q, w = oracle.prepare_query(weights_np, synth.make_hidden(wl)[:1], synth.make_positions(wl)[:1],
                                oracle.OracleConfig())
    g = torch.Generator(device="cuda").manual_seed(2026)
    ck = torch.empty((1, N, RECORD), dtype=torch.uint8, device="cuda")
    step = 1 << 22
    for i in range(0, N, step):
        codes = torch.randint(0, 256, (step, 128), generator=g, device="cuda", dtype=torch.uint8)
        ck[0, i:i + step, :128] = codes & 0xBF
        mag = torch.rand(step, generator=g, device="cuda") * 0.18 + 0.02
        sign = torch.randint(0, 2, (step,), generator=g, device="cuda").float() * 2 - 1
        ck[0, i:i + step, 128:] = (mag * sign).contiguous().view(torch.uint8).view(step, 4)
    qd = torch.from_numpy(q.astype(np.float32)).cuda()
    wd = torch.from_numpy(w.astype(np.float32)).cuda()
    yield r, ck, qd, wd, q, w
    r.close()


def sample_chunks():
    rng = np.random.default_rng(7)
    c0 = (1 << 32) // RECORD                         # its record starts below 2^32, the next one's above
    edges = [0, 1, 15, 16, 17, N - 17, N - 16, N - 2, N - 1, c0 - 1, c0, c0 + 1, c0 + 2]
    for k in (1, 2, 511, 512, 1023):                 # wave shares of 65536 chunks on 1024 waves
        edges += [k * 65536 - 1, k * 65536]
    return np.unique(np.concatenate([np.array(edges, np.int64), rng.integers(0, N, 200)]))


@pytest.mark.parametrize("fp8", [False, True])
def test_max_n_scores_on_sampled_chunks(big, fp8):
    r, ck, qd, wd, q, w = big
    s, p = r.score(qd, wd, ck, None, "max", per_layer=True, fp8=fp8)
    idx = sample_chunks()
    it = torch.from_numpy(idx).cuda()
    recs = ck[0].index_select(0, it).cpu().numpy()[None]
    s_h = s[0].index_select(0, it).cpu().numpy()[None]
    p_h = p[:, 0].index_select(1, it).cpu().numpy()[:, None]
    per_ref, ens_ref = oracle.score_row(recs[0], q[:, 0], w[:, 0], len(idx), "max")
    e = max(max_score_err(s_h, ens_ref[None]), max_score_err(p_h, per_ref[:, None]))
    report(f"N = 2^26, {len(idx)} sampled chunks ({'fp8' if fp8 else 'f16'})", max_abs=e)
    assert e <= SCORE_TOL


def test_max_n_topk_exact(big):
    r, ck, qd, wd, q, w = big
    s = r.score(qd, wd, ck, None, "max")
    m = r.keep_topk(s, 512)
    torch.cuda.synchronize()
    own = oracle.select_topk(s[0].cpu().numpy().astype(np.float64), N, 512)
    assert np.array_equal(m[0].cpu().numpy().astype(np.uint8), own)


def test_max_n_threshold_in_the_score_pass(big):
    r, ck, qd, wd, q, w = big
    s, m = r.score_select(qd, wd, ck, None, "mean", threshold=0.5)
    torch.cuda.synchronize()
    s_h = s[0].cpu().numpy().astype(np.float64)
    own = oracle.select_threshold(s_h, N, 0.5)
    assert np.array_equal(m[0].cpu().numpy().astype(np.uint8), own)
    idx = sample_chunks()
    recs = ck[0].index_select(0, torch.from_numpy(idx).cuda()).cpu().numpy()
    _, ens_ref = oracle.score_row(recs, q[:, 0], w[:, 0], len(idx), "mean")
    e = max_score_err(s_h[idx], ens_ref)
    report(f"N = 2^26, mean + threshold, {len(idx)} sampled chunks", max_abs=e, kept=int(own.sum()))
    assert e <= SCORE_TOL


def test_max_n_resident_delta(big):
    """Resident set and recall delta between two top-4096 masks of the row
    (the max and the mean ensemble's), against the oracle's lists."""
    r, ck, qd, wd, q, w = big
    cur = r.keep_topk(r.score(qd, wd, ck, None, "max"), 4096)
    prev = r.keep_topk(r.score(qd, wd, ck, None, "mean"), 4096)
    res, ent, lea = r.resident_delta(cur, prev, cap=8192)
    ref = oracle.resident_delta(cur[0].cpu().numpy(), prev[0].cpu().numpy())
    for got, want, name in zip((res[0], ent[0], lea[0]), ref, ("resident", "entering", "leaving")):
        assert np.array_equal(got.cpu().numpy().astype(np.int64), want), name
    report("N = 2^26, resident delta", resident=len(ref[0]), entering=len(ref[1]), leaving=len(ref[2]))


def test_max_n_subset_topk(big):
    """Top-512 of the mean-ensemble scores within the max ensemble's top-32768
    chunks (the scan + finish path's longest list), against the oracle."""
    r, ck, qd, wd, q, w = big
    s_max = r.score(qd, wd, ck, None, "max")
    s_mean = r.score(qd, wd, ck, None, "mean")
    (res,), _, _ = r.resident_delta(r.keep_topk(s_max, 32768), None, cap=32768)
    subset = res.reshape(1, -1).contiguous()
    out, n_out = r.topk_in_subset(s_mean, subset, 512)
    torch.cuda.synchronize()
    want = oracle.select_topk_subset(s_mean[0].cpu().numpy(), subset[0].cpu().numpy(), 512)
    assert int(n_out[0]) == len(want) == 512
    assert np.array_equal(out[0].cpu().numpy().astype(np.int64), want)
