"""Attention-logit masking (fm_mask_logits) against the oracle, bit for bit:
fp32 and bf16 logits, assorted (B, R, N) including rows that start
unaligned and ragged tails, masks of every density with non-0/1 bytes, a
keep mask from the real selection, and the softmax property (a masked chunk
gets no attention weight)."""

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


def run_raw(retr, logits, mask_u8):
    """fm_mask_logits through the C ABI on a uint8 mask."""
    from sparse_attention_chunk_amd import _lib
    B, R, N = logits.shape
    dt = _lib.FM_DTYPE_F32 if logits.dtype == torch.float32 else _lib.FM_DTYPE_BF16
    _lib.fm_mask_logits(retr.ctx, logits, dt, B, R, N, mask_u8)
    torch.cuda.synchronize()
    return logits


def bits(t):
    t = t.cpu()
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)).numpy()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("B,R,N", [(2, 3, 1), (2, 4, 17), (3, 8, 4096), (2, 5, 70001), (1, 2, 262144),
                                   (5, 6, 8200), (5, 9, 65536)])
def test_random_masks_bit_exact(retr, dtype, B, R, N):
    rng = np.random.default_rng(B * 100 + R * 10 + N)
    logits = torch.from_numpy(rng.normal(size=(B, R, N)).astype(np.float32)).to(dtype)
    dens = [0.0, 1.0, 0.002, 0.3, 0.9][:B]
    mask = np.stack([(rng.uniform(size=N) < d) for d in dens]).astype(np.uint8)
    mask *= rng.integers(1, 256, size=mask.shape).astype(np.uint8)  # any non-zero byte keeps
    got = run_raw(retr, logits.cuda(), torch.from_numpy(mask).cuda())
    ref = logits.clone()
    for b in range(B):
        m = torch.from_numpy(oracle.mask_logits(np.zeros((1, N)), mask[b])[0])
        ref[b][:, torch.isneginf(m)] = float("-inf")
    assert np.array_equal(bits(got), bits(ref))


def test_softmax_weight_of_masked_chunks_is_zero(retr):
    """Logits masked with a real top-512 keep mask: softmax puts no weight on
    dropped chunks and matches the softmax over the kept ones."""
    wl = synth.WORKLOADS[1]
    hidden = torch.from_numpy(synth.make_hidden(wl)).cuda()
    pos = torch.from_numpy(synth.make_positions(wl)).cuda()
    comp = torch.from_numpy(synth.make_comp_k(wl)).cuda()
    keep = retr.select_topk(hidden, comp, pos, top_k=512)
    rng = np.random.default_rng(9)
    logits_np = rng.normal(size=(1, 64, wl.n_chunks)).astype(np.float32)
    out = retr.mask_logits(torch.from_numpy(logits_np).cuda(), keep).cpu().numpy().astype(np.float64)
    k = keep.cpu().numpy()[0]
    assert np.array_equal(out[0], oracle.mask_logits(logits_np[0].astype(np.float64), k))
    e = np.exp(out[0] - out[0].max(axis=1, keepdims=True))
    p = e / e.sum(axis=1, keepdims=True)
    x = logits_np[0][:, k].astype(np.float64)
    ek = np.exp(x - x.max(axis=1, keepdims=True))
    assert np.all(p[:, ~k] == 0) and np.allclose(p[:, k], ek / ek.sum(axis=1, keepdims=True), rtol=1e-12, atol=0)
    report("mask_logits top-512 softmax", kept=int(k.sum()))


def test_argument_errors(retr):
    from sparse_attention_chunk_amd import _lib
    L = _lib.LIB
    x = torch.zeros((2, 3, 100), device="cuda")
    m = torch.zeros((2, 100), dtype=torch.uint8, device="cuda")
    assert L.fm_mask_logits(retr.ctx, x.data_ptr(), 7, 2, 3, 100, m.data_ptr(), None) == _lib.FM_EINVAL
    assert L.fm_mask_logits(retr.ctx, x.data_ptr(), 0, 2, -1, 100, m.data_ptr(), None) == _lib.FM_EINVAL
    assert L.fm_mask_logits(retr.ctx, None, 0, 2, 3, 100, m.data_ptr(), None) == _lib.FM_EINVAL
    assert L.fm_mask_logits(retr.ctx, x.data_ptr() + 2, 0, 2, 3, 100, m.data_ptr(), None) == _lib.FM_EINVAL
    assert L.fm_mask_logits(retr.ctx, x.data_ptr(), 0, 65, 3, 100, m.data_ptr(), None) == _lib.FM_EINVAL
    assert L.fm_mask_logits(retr.ctx, None, 0, 2, 0, 100, None, None) == _lib.FM_OK
    with pytest.raises(ValueError):
        retr.mask_logits(torch.zeros((2, 3, 100), dtype=torch.float16, device="cuda"), m.bool())
