"""The hot path under HIP graph capture: fm_prepare_query + fm_score +
fm_select_topk, fm_score_threshold (the threshold mask written by the score
pass), and the calls around it (fm_score_fp8, fm_resident_delta
against the previous cycle's mask, and the decode-step calls
fm_select_topk_subset and fm_mask_logits), captured once and replayed
several times, with eager work and synchronisations between the replays;
every replay must equal the eager result bit for bit.  The calls allocate
nothing and never synchronise, so they can be captured."""

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def retr():
    import sparse_attention_chunk_amd as fm
    r = fm.FlashMemoryRetriever(fm.weights_to_device(synth.make_weights()), max_batch=8, max_n=65536)
    yield r
    r.close()


def test_graph_replays_match_eager(retr):
    from sparse_attention_chunk_amd import _lib
    wl = synth.WORKLOADS[3]
    rows = [1, 4]
    B, N = len(rows), 65536
    hidden = torch.from_numpy(synth.make_hidden(wl)[rows]).cuda()
    pos = torch.from_numpy(synth.make_positions(wl)[rows]).cuda()
    comp = torch.from_numpy(synth.make_comp_k(wl, rows=rows)[:, :N].copy()).cuda()

    q = torch.empty((3, B, 64, 128), device="cuda")
    w = torch.empty((3, B, 64), device="cuda")
    scores = torch.empty((B, N), device="cuda")
    mask = torch.empty((B, N), dtype=torch.bool, device="cuda")
    cap, K = 4096, 512
    sub = torch.stack([torch.arange(i, N, N // cap, dtype=torch.int32, device="cuda")[:cap] for i in range(B)])
    step = torch.rand((B, N), generator=torch.Generator(device="cuda").manual_seed(3), device="cuda")
    out = torch.empty((B, K), dtype=torch.int32, device="cuda")
    n_out = torch.empty((B,), dtype=torch.int32, device="cuda")
    logits = torch.empty((B, 8, N), dtype=torch.bfloat16, device="cuda")
    logits_src = torch.randn((B, 8, N), generator=torch.Generator(device="cuda").manual_seed(4), device="cuda",
                             dtype=torch.bfloat16)
    scores8 = torch.empty((B, N), device="cuda")
    prev = (torch.rand((B, N), generator=torch.Generator(device="cuda").manual_seed(5), device="cuda") < 0.01)
    prev = prev.to(torch.uint8)
    rcap = 2048
    res = torch.empty((B, rcap), dtype=torch.int32, device="cuda")
    ent = torch.empty((B, rcap), dtype=torch.int32, device="cuda")
    lea = torch.empty((B, rcap), dtype=torch.int32, device="cuda")
    n_res, n_ent, n_lea = (torch.empty((B,), dtype=torch.int32, device="cuda") for _ in range(3))
    scores_t = torch.empty((B, N), device="cuda")
    mask_t = torch.empty((B, N), dtype=torch.bool, device="cuda")

    def body(stream):
        sh = stream.cuda_stream
        _lib.fm_prepare_query(retr.ctx, hidden, pos, B, q, w, sh)
        _lib.fm_score(retr.ctx, q, w, comp, B, N, None, _lib.FM_ENSEMBLE_MAX, scores, None, sh)
        _lib.fm_select_topk(retr.ctx, scores, B, N, None, K, mask, sh)
        _lib.fm_score_threshold(retr.ctx, q, w, comp, B, N, None, _lib.FM_ENSEMBLE_MEAN, 0.5, scores_t, mask_t, None,
                                sh)
        _lib.fm_score_fp8(retr.ctx, q, w, comp, B, N, None, _lib.FM_ENSEMBLE_MAX, scores8, None, sh)
        _lib.fm_resident_delta(retr.ctx, prev, mask, B, N, rcap, res, n_res, ent, n_ent, lea, n_lea, sh)
        _lib.fm_select_topk_subset(retr.ctx, step, B, N, sub, None, cap, K, out, n_out, sh)
        logits.copy_(logits_src)
        _lib.fm_mask_logits(retr.ctx, logits, _lib.FM_DTYPE_BF16, B, 8, N, mask, sh)

    def snapshot():
        torch.cuda.synchronize()
        return [t.clone() for t in (q, w, scores, mask, out, n_out, logits, scores8, res, n_res, ent, n_ent, lea,
                                    n_lea, scores_t, mask_t)]

    def clear():
        # The lists are written only up to their counts: their tails stay as cleared.
        for t in (q, w, scores, out, n_out, logits, scores8, res, n_res, ent, n_ent, lea, n_lea, scores_t):
            t.zero_()
        for t in (mask, mask_t):
            t.fill_(False)

    clear()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        body(s)
    torch.cuda.current_stream().wait_stream(s)
    eager = snapshot()
    assert int(eager[3].sum()) == B * K

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body(torch.cuda.current_stream())
    for rep in range(4):
        clear()
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        for a, b in zip(got, eager):
            assert torch.equal(a, b), f"replay {rep}"
        # eager work between replays
        _ = (scores * 2).sum().item()
