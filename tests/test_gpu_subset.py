"""Per-step top-K within each row's resident set (fm_select_topk_subset)
against the oracle: exact chosen lists and counts on random subsets (sorted
and unsorted, with out-of-range entries, ragged lengths, tied and -inf
scores), subsets held in LDS and gathered per pass, the whole row as the
subset, a retrieval cycle feeding a decode step, and argument errors."""

import numpy as np
import pytest
import torch

import oracle
import synth
from fm_cases import report

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def retr():
    import sparse_attention_chunk_amd as fm
    r = fm.FlashMemoryRetriever(fm.weights_to_device(synth.make_weights()), max_batch=64, max_n=1 << 18)
    yield r
    r.close()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def make_case(seed, B, N, cap, order="sorted", bad=0):
    """Scores with ties and some -inf, subsets of distinct chunk indices
    (ascending or shuffled), optionally with out-of-range entries, and
    ragged per-row lengths."""
    rng = np.random.default_rng(seed)
    scores = (rng.integers(0, 256, (B, N)) / 256.0).astype(np.float32)
    scores[rng.uniform(size=(B, N)) < 0.01] = -np.inf
    subset = np.full((B, cap), -9, np.int32)
    n_sub = np.zeros(B, np.int32)
    for b in range(B):
        n = [cap, cap // 2, 1, 0, cap - 3][b % 5]
        n = max(0, min(n, cap, N))
        pick = rng.choice(N, size=n, replace=False)
        pick = np.sort(pick) if order == "sorted" else rng.permutation(pick)
        if bad and n:
            where = rng.choice(n, size=min(bad, n), replace=False)
            pick[where] = rng.choice([-1, -7, N, N + 5], size=len(where))
        subset[b, :n] = pick
        n_sub[b] = n
    return scores, subset, n_sub


def check(retr, scores, subset, n_sub, top_k, with_count=True):
    s, sub = torch.from_numpy(scores).cuda(), torch.from_numpy(subset).cuda()
    ns = torch.from_numpy(n_sub).cuda() if with_count else None
    out, n_out = retr.topk_in_subset(s, sub, top_k, ns)
    out, n_out = host(out), host(n_out)
    for b in range(scores.shape[0]):
        m = int(n_sub[b]) if with_count else subset.shape[1]
        want = oracle.select_topk_subset(scores[b], subset[b, :m], top_k)
        assert n_out[b] == len(want), (b, n_out[b], len(want))
        assert np.array_equal(out[b, :len(want)], want), b
    return n_out


@pytest.mark.parametrize("B,N,cap,order,bad", [
    (3, 1000, 17, "sorted", 0),
    (5, 70000, 5000, "sorted", 3),
    (5, 50000, 3000, "shuffled", 2),
    (2, 262144, 32768, "sorted", 0),     # the longest list of the tile scan + finish path
    (2, 262144, 65536, "sorted", 5),     # longer lists: keys gathered again in every pass
    (3, 4096, 4096, "sorted", 0),
    (3, 70000, 8192, "shuffled", 4),     # the longest list of the one-launch path
    (3, 70000, 8193, "sorted", 2),       # the shortest of the tile scan + finish path
])
def test_random_subsets_exact(retr, B, N, cap, order, bad):
    scores, subset, n_sub = make_case(B * 7 + cap, B, N, cap, order, bad)
    for k in (0, 1, 512, cap + 5):
        check(retr, scores, subset, n_sub, k)
    report(f"subset top-k B={B} N={N} cap={cap} {order}", rows=B)


@pytest.mark.parametrize("levels,k", [(4, 512), (64, 512), (100000, 7000), (3, 20000)])
def test_heavy_ties_fall_back_to_whole_list_selection(retr, levels, k):
    """Lists of up to 32768 entries take the tile scan + finish; heavy ties
    at the cut-off (few distinct scores) overflow its candidate lists and
    fall back to a radix selection over the whole list.  Both must give the
    exact result."""
    rng = np.random.default_rng(levels + k)
    B, N, cap = 3, 262144, 32768
    scores = (rng.integers(0, levels, (B, N)) / levels).astype(np.float32)
    subset = np.stack([np.sort(rng.choice(N, cap, replace=False)) for _ in range(B)]).astype(np.int32)
    n_sub = np.array([cap, 30001, 9000], np.int32)
    check(retr, scores, subset, n_sub, k)


def test_small_context_lists_longer_than_the_row():
    """A small context (max_n 8192) with lists longer than N, padded with
    out-of-range entries, in list order and shuffled."""
    import sparse_attention_chunk_amd as fm
    r = fm.FlashMemoryRetriever(fm.weights_to_device(synth.make_weights()), max_batch=4, max_n=8192)
    try:
        rng = np.random.default_rng(21)
        B, N, cap = 3, 8000, 20000
        scores = (rng.integers(0, 5000, (B, N)) / 5000.0).astype(np.float32)
        subset = np.full((B, cap), -1, np.int32)
        for b in range(B):
            vals = np.concatenate([rng.permutation(N), rng.integers(N, 3 * N, cap - N)])
            subset[b] = rng.permutation(vals)[:cap] if b else vals
        for k in (1, 512, 6000):
            check(r, scores, subset, np.array([cap, 15000, 9000], np.int32), k)
    finally:
        r.close()


def test_without_counts_uses_cap(retr):
    scores, subset, n_sub = make_case(3, 2, 9000, 1200)
    subset[:, :] = np.stack([np.sort(np.random.default_rng(b).choice(9000, 1200, replace=False))
                             for b in range(2)]).astype(np.int32)
    check(retr, scores, subset, np.full(2, 1200, np.int32), 300, with_count=False)


def test_whole_row_subset_matches_row_top_k(retr):
    """The subset of every chunk chooses what the row's top-K keeps."""
    rng = np.random.default_rng(11)
    B, N = 3, 20000
    scores = (rng.integers(0, 1000, (B, N)) / 1000.0).astype(np.float32)
    s = torch.from_numpy(scores).cuda()
    sub = torch.arange(N, dtype=torch.int32, device="cuda").repeat(B, 1).contiguous()
    for k in (1, 512, 7000):
        out, n_out = retr.topk_in_subset(s, sub, k)
        mask = host(retr.keep_topk(s, k))
        o, n = host(out), host(n_out)
        for b in range(B):
            assert n[b] == k and np.array_equal(o[b], np.flatnonzero(mask[b]))


def test_decode_step_within_the_recalled_set(retr):
    """A retrieval cycle keeps 4096 chunks per row; a decode step's top-512
    then runs over that resident set with the step's own scores."""
    wl = synth.WORKLOADS[3]
    rows = [0, 9]
    hidden = torch.from_numpy(synth.make_hidden(wl)[rows]).cuda()
    pos = torch.from_numpy(synth.make_positions(wl)[rows]).cuda()
    comp = torch.from_numpy(synth.make_comp_k(wl, rows=rows)[:, :65536].copy()).cuda()
    scores = retr.ensemble(hidden, comp, pos, "max")
    keep = retr.keep_topk(scores, 4096)
    resident, _, _ = retr.resident_delta(keep)
    cap = 4096
    sub = torch.stack([r for r in resident]).to(torch.int32).contiguous()
    step = torch.from_numpy(np.random.default_rng(5).uniform(size=(2, 65536)).astype(np.float32)).cuda()
    out, n_out = retr.topk_in_subset(step, sub, 512)
    o, n, st, sb = host(out), host(n_out), host(step), host(sub)
    for b in range(2):
        want = oracle.select_topk_subset(st[b], sb[b], 512)
        assert n[b] == 512 and np.array_equal(o[b], want)
        assert np.all(host(keep)[b][o[b]])  # every chosen chunk is resident
    report("subset top-512 after a 4096-chunk recall", cap=cap)


def test_argument_errors(retr):
    from sparse_attention_chunk_amd import _lib
    L = _lib.LIB
    ctx = retr.ctx
    s = torch.zeros((2, 100), device="cuda")
    sub = torch.zeros((2, 10), dtype=torch.int32, device="cuda")
    out = torch.zeros((2, 5), dtype=torch.int32, device="cuda")
    n = torch.zeros((2,), dtype=torch.int32, device="cuda")
    P = lambda t: t.data_ptr()  # noqa: E731
    assert L.fm_select_topk_subset(ctx, P(s), 2, 100, P(sub), None, -1, 5, P(out), P(n), None) == _lib.FM_EINVAL
    assert L.fm_select_topk_subset(ctx, P(s), 2, 100, P(sub), None, 10, -1, P(out), P(n), None) == _lib.FM_EINVAL
    assert L.fm_select_topk_subset(ctx, P(s), 2, 100, None, None, 10, 5, P(out), P(n), None) == _lib.FM_EINVAL
    assert L.fm_select_topk_subset(ctx, P(s), 2, 100, P(sub), None, 10, 5, None, P(n), None) == _lib.FM_EINVAL
    assert L.fm_select_topk_subset(ctx, P(s), 2, 100, P(sub), None, 10, 5, P(out), None, None) == _lib.FM_EINVAL
    assert L.fm_select_topk_subset(ctx, P(s), 65, 100, P(sub), None, 10, 5, P(out), P(n), None) == _lib.FM_EINVAL
    assert L.fm_select_topk_subset(ctx, P(s) + 2, 2, 100, P(sub), None, 10, 5, P(out), P(n), None) == _lib.FM_EINVAL
    assert L.fm_select_topk_subset(ctx, None, 0, 0, None, None, 0, 0, None, None, None) == _lib.FM_OK
    # cap 0 and top_k 0: only the counts are written
    n.fill_(-3)
    assert L.fm_select_topk_subset(ctx, P(s), 2, 100, None, None, 0, 0, None, P(n), None) == _lib.FM_OK
    assert list(host(n)) == [0, 0]
