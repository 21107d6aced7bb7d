"""Two contexts on two streams at once (a context serves one stream at a
time): consecutive passes pipelined so that pass i's top-K runs on a second
stream, with its own context, while pass i+1's query preparation and score
run on the first.  Scores and masks are double-buffered; every pass must
equal the same pass run alone on one stream, bit for bit."""

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def test_two_contexts_pipelined_over_two_streams_match_one_stream():
    import sparse_attention_chunk_amd as fm
    from sparse_attention_chunk_amd import _lib as L
    rows = [0, 3, 5]
    B, N, K = len(rows), 32768, 512
    weights = fm.weights_to_device(synth.make_weights())
    ra = fm.FlashMemoryRetriever(weights, max_batch=B, max_n=N)
    rb = fm.FlashMemoryRetriever(weights, max_batch=B, max_n=N)
    try:
        wl3 = synth.WORKLOADS[3]
        comp = torch.from_numpy(synth.make_comp_k(wl3, rows=rows)[:, :N].copy()).cuda()
        hid_all = torch.from_numpy(synth.make_hidden(wl3)).cuda()
        pos_all = torch.from_numpy(synth.make_positions(wl3)).cuda()
        # Four passes over different hidden rows (so consecutive passes differ).
        passes = [(hid_all[4 * i:4 * i + B].contiguous(), pos_all[4 * i:4 * i + B].contiguous()) for i in range(4)]
        q = torch.empty((3, B, 64, 128), device="cuda")
        w = torch.empty((3, B, 64), device="cuda")

        sa = torch.cuda.current_stream()
        ref = []
        for hid, pos in passes:
            sc = torch.empty((B, N), device="cuda")
            mk = torch.empty((B, N), dtype=torch.bool, device="cuda")
            L.fm_prepare_query(ra.ctx, hid, pos, B, q, w, sa.cuda_stream)
            L.fm_score(ra.ctx, q, w, comp, B, N, None, L.FM_ENSEMBLE_MAX, sc, None, sa.cuda_stream)
            L.fm_select_topk(ra.ctx, sc, B, N, None, K, mk, sa.cuda_stream)
            ref.append((sc, mk))
        torch.cuda.synchronize()

        sb = torch.cuda.Stream()
        scores = [torch.full((B, N), 7.0, device="cuda") for _ in range(2)]
        masks = [torch.zeros((B, N), dtype=torch.bool, device="cuda") for _ in range(2)]
        ev_score = [torch.cuda.Event() for _ in range(2)]
        ev_sel = [torch.cuda.Event() for _ in range(2)]
        for e in ev_sel:
            e.record(sa)
        got = []
        for i, (hid, pos) in enumerate(passes):
            b = i & 1
            L.fm_prepare_query(ra.ctx, hid, pos, B, q, w, sa.cuda_stream)
            sa.wait_event(ev_sel[b])
            if i >= 2:  # the pass that last used buffer b is complete: keep a copy of its outputs
                got.append((scores[b].clone(), masks[b].clone()))
            L.fm_score(ra.ctx, q, w, comp, B, N, None, L.FM_ENSEMBLE_MAX, scores[b], None, sa.cuda_stream)
            ev_score[b].record(sa)
            sb.wait_event(ev_score[b])
            L.fm_select_topk(rb.ctx, scores[b], B, N, None, K, masks[b], sb.cuda_stream)
            ev_sel[b].record(sb)
        torch.cuda.synchronize()
        got += [(scores[0].clone(), masks[0].clone()), (scores[1].clone(), masks[1].clone())]
        assert len(got) == len(ref)
        for i, ((gs, gm), (rs, rm)) in enumerate(zip(got, ref)):
            assert torch.equal(gs, rs), f"scores of pass {i}"
            assert torch.equal(gm, rm), f"mask of pass {i}"
            assert int(gm.sum()) == B * K
        assert not torch.equal(ref[0][1], ref[1][1])  # the passes differ
    finally:
        ra.close()
        rb.close()
