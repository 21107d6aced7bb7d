"""fm_select_topk_static (no context, no allocation: its scratch is a static
device array) through the C ABI, against fm_select_topk on the same scores:
masks identical, on two calls in a row, the second smaller than the first
(the scratch keeps the first call's contents), then on rows short enough
for the one-launch path."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _scores(B, N, seed, ties):
    g = torch.Generator(device="cuda").manual_seed(seed)
    s = torch.rand((B, N), generator=g, device="cuda")
    if ties:
        s = torch.round(s * 1000) / 1000
    return s


def _both(ctx, scores, valid_n, k):
    from sparse_attention_chunk_amd import _lib
    B, N = scores.shape
    m_ctx = torch.ones((B, N), dtype=torch.uint8, device="cuda")
    m_static = torch.ones((B, N), dtype=torch.uint8, device="cuda")
    _lib.fm_select_topk(ctx, scores, B, N, valid_n, k, m_ctx)
    _lib.fm_select_topk_static(scores, B, N, valid_n, k, m_static)
    torch.cuda.synchronize()
    return m_ctx, m_static


def test_static_topk_matches_the_context_call_twice_second_smaller():
    import sparse_attention_chunk_amd as fm
    import synth
    from sparse_attention_chunk_amd import _lib
    r = fm.FlashMemoryRetriever(fm.weights_to_device(synth.make_weights()), max_batch=30, max_n=262144)
    try:
        # 1: the full-size launch (B=30, N=262144, top-512)
        s1 = _scores(30, 262144, 1, ties=False)
        a, b = _both(r.ctx, s1, None, 512)
        assert torch.equal(a, b) and int(b.sum()) == 30 * 512
        # 2: smaller, ragged, heavy ties, N not a multiple of 16 (rows longer
        # than 8192 chunks: the scan + finish path on the static scratch)
        s2 = _scores(4, 20003, 2, ties=True)
        vn = torch.tensor([20003, 16000, 17, 0], dtype=torch.int32, device="cuda")
        for k in (1, 17, 600):
            a, b = _both(r.ctx, s2, vn, k)
            assert torch.equal(a, b), k
            counts = b.sum(dim=1).cpu().numpy()
            assert list(counts) == [min(k, 20003), min(k, 16000), min(k, 17), 0]
        # 3: short rows (one launch, no scratch needed)
        s3 = _scores(4, 5003, 3, ties=True)
        vn3 = torch.tensor([5003, 4000, 17, 0], dtype=torch.int32, device="cuda")
        for k in (1, 600):
            a, b = _both(r.ctx, s3, vn3, k)
            assert torch.equal(a, b), k
            assert list(b.sum(dim=1).cpu().numpy()) == [min(k, 5003), min(k, 4000), min(k, 17), 0]
        # oversize: rejected, nothing launched
        big = torch.empty((65, 16), device="cuda")
        with pytest.raises(_lib.FmError) as e:
            _lib.fm_select_topk_static(big, 65, 262144, None, 512, big)
        assert e.value.status == _lib.FM_EINVAL
    finally:
        r.close()
