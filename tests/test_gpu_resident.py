"""Resident set and recall delta (fm_resident_delta) against the oracle:
exact index lists and counts on random masks of assorted shapes and
densities, with and without a previous mask, non-0/1 mask bytes, capped
lists, two cycles of the real selection, and argument errors."""

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


def run_raw(retr, mask_u8, prev_u8, cap):
    """fm_resident_delta through the C ABI on uint8 masks."""
    from sparse_attention_chunk_amd import _lib
    B, N = mask_u8.shape
    dev = mask_u8.device
    lists = [torch.full((B, max(cap, 1)), -7, dtype=torch.int32, device=dev) for _ in range(3)]
    counts = [torch.full((B,), -7, dtype=torch.int32, device=dev) for _ in range(3)]
    _lib.fm_resident_delta(retr.ctx, prev_u8, mask_u8, B, N, cap, lists[0], counts[0], lists[1], counts[1],
                           lists[2], counts[2])
    return [host(x) for x in lists], [host(c) for c in counts]


def check_rows(mask, prev, lists, counts, cap):
    for b in range(mask.shape[0]):
        want = oracle.resident_delta(mask[b], None if prev is None else prev[b])
        for k in range(3):
            assert counts[k][b] == len(want[k]), (b, k)
            m = min(len(want[k]), cap)
            assert np.array_equal(lists[k][b, :m], want[k][:m]), (b, k)


@pytest.mark.parametrize("B,N", [(3, 1), (2, 15), (2, 16), (3, 4097), (5, 70000), (4, 131073)])
def test_random_masks_exact(retr, B, N):
    rng = np.random.default_rng(B * 1000 + N)
    dens = [0.0, 1.0, 0.002, 0.3, 0.5][:B] + [0.1] * max(0, B - 5)
    mask = np.stack([(rng.uniform(size=N) < d) for d in dens]).astype(np.uint8)
    prev = np.stack([(rng.uniform(size=N) < d) for d in reversed(dens)]).astype(np.uint8)
    md, pd = torch.from_numpy(mask).cuda(), torch.from_numpy(prev).cuda()
    for p, pdev in ((None, None), (prev, pd)):
        lists, counts = run_raw(retr, md, pdev, N)
        check_rows(mask, p, lists, counts, N)
    report(f"resident_delta B={B} N={N}", rows=B)


def test_nonzero_bytes_count_as_kept(retr):
    rng = np.random.default_rng(5)
    N = 5003
    mask = rng.integers(0, 4, (2, N)).astype(np.uint8) * (rng.uniform(size=(2, N)) < 0.3)
    mask = mask.astype(np.uint8)
    mask[0, :20] = np.array([0, 1, 2, 255] * 5, np.uint8)
    prev = (rng.integers(0, 256, (2, N)) * (rng.uniform(size=(2, N)) < 0.3)).astype(np.uint8)
    lists, counts = run_raw(retr, torch.from_numpy(mask).cuda(), torch.from_numpy(prev).cuda(), N)
    check_rows(mask, prev, lists, counts, N)


def test_cap_truncates_lists_and_keeps_full_counts(retr):
    rng = np.random.default_rng(6)
    N = 9000
    mask = (rng.uniform(size=(3, N)) < 0.2).astype(np.uint8)
    prev = (rng.uniform(size=(3, N)) < 0.2).astype(np.uint8)
    for cap in (0, 1, 100, 1700):
        lists, counts = run_raw(retr, torch.from_numpy(mask).cuda(), torch.from_numpy(prev).cuda(), cap)
        check_rows(mask, prev, lists, counts, cap)
        if cap > 0:  # nothing written past cap
            for k in range(3):
                assert np.all(lists[k][:, cap:] == -7)


def test_two_cycles_of_the_real_selection(retr):
    """Masks of two retrieval cycles (top-512 of the same keys scored for two
    positions of the decode token): the delta of the GPU masks is exact, and
    the python wrapper returns the same lists."""
    wl = synth.WORKLOADS[3]
    rows = [0, 7]
    hidden = torch.from_numpy(synth.make_hidden(wl)[rows]).cuda()
    comp = torch.from_numpy(synth.make_comp_k(wl, rows=rows)[:, :65536].copy()).cuda()
    masks = []
    for shift in (0, 64 * 4):
        pos = torch.from_numpy(synth.make_positions(wl)[rows] + shift).cuda()
        s = retr.ensemble(hidden, comp, pos, "max")
        masks.append(retr.keep_topk(s, 512))
    prev, cur = masks
    res, ent, lea = retr.resident_delta(cur, prev)
    pm, cm = host(prev).astype(np.uint8), host(cur).astype(np.uint8)
    for b in range(len(rows)):
        want = oracle.resident_delta(cm[b], pm[b])
        assert np.array_equal(host(res[b]), want[0])
        assert np.array_equal(host(ent[b]), want[1])
        assert np.array_equal(host(lea[b]), want[2])
        assert len(want[0]) == 512
    report("resident_delta two cycles", entering=float(np.mean([len(host(e)) for e in ent])))


def test_argument_errors(retr):
    from sparse_attention_chunk_amd import _lib
    m = torch.zeros((2, 100), dtype=torch.uint8, device="cuda")
    out = torch.zeros((2, 100), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((2,), dtype=torch.int32, device="cuda")
    L = _lib.LIB
    ctx = retr.ctx
    assert L.fm_resident_delta(ctx, None, m.data_ptr(), 2, 100, -1, out.data_ptr(), cnt.data_ptr(), None, None, None,
                               None, None) == _lib.FM_EINVAL
    assert L.fm_resident_delta(ctx, None, m.data_ptr(), 2, 100, 100, out.data_ptr(), cnt.data_ptr(), out.data_ptr(),
                               None, None, None, None) == _lib.FM_EINVAL
    assert L.fm_resident_delta(ctx, None, None, 2, 100, 100, out.data_ptr(), cnt.data_ptr(), None, None, None, None,
                               None) == _lib.FM_EINVAL
    assert L.fm_resident_delta(ctx, None, None, 0, 0, 0, None, None, None, None, None, None, None) == _lib.FM_OK


def test_many_calls_in_a_row_on_one_context(retr):
    """Back-to-back calls of different shapes on one context: no call sees
    another's intermediate counts."""
    rng = np.random.default_rng(78)
    for it, (B, N) in enumerate([(4, 262144), (2, 5000), (4, 262144), (3, 77777), (1, 4096), (4, 262144)]):
        mask = (rng.uniform(size=(B, N)) < 0.01 * (it + 1)).astype(np.uint8)
        prev = (rng.uniform(size=(B, N)) < 0.02).astype(np.uint8)
        lists, counts = run_raw(retr, torch.from_numpy(mask).cuda(), torch.from_numpy(prev).cuda(), N)
        check_rows(mask, prev, lists, counts, N)
