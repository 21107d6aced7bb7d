"""Error conventions of the C ABI on a live context: every failing call
returns its status before enqueueing anything, so outputs keep their
sentinel contents."""

import ctypes

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import sparse_attention_chunk_amd as fm
    from sparse_attention_chunk_amd import _lib
    r = fm.FlashMemoryRetriever(fm.weights_to_device(synth.make_weights()), max_batch=4, max_n=1000)
    yield r, _lib
    r.close()


def test_argument_errors_enqueue_nothing(env):
    r, L = env
    lib, ctx = L.LIB, r.ctx
    EINVAL = L.FM_EINVAL
    B, N = 2, 100
    q = torch.zeros((3, B, 64, 128), device="cuda")
    w = torch.zeros((3, B, 64), device="cuda")
    ck = torch.zeros((B, N, 132), dtype=torch.uint8, device="cuda")
    ck_big = torch.zeros((B * N * 132 + 16,), dtype=torch.uint8, device="cuda")
    scores = torch.full((B, N), 7.0, device="cuda")
    mask = torch.full((B, N), 9, dtype=torch.uint8, device="cuda")
    hidden = torch.zeros((B, 4096), device="cuda")
    pos = torch.zeros((B,), dtype=torch.int64, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    P = L.ptr

    cases = [
        lib.fm_score(ctx, None, P(w), P(ck), B, N, None, 0, P(scores), None, s),             # null q
        lib.fm_score(ctx, P(q), P(w), None, B, N, None, 0, P(scores), None, s),              # null comp_k
        lib.fm_score(ctx, P(q), P(w), P(ck), 5, N, None, 0, P(scores), None, s),             # B > max_batch
        lib.fm_score(ctx, P(q), P(w), P(ck), -1, N, None, 0, P(scores), None, s),            # B < 0
        lib.fm_score(ctx, P(q), P(w), P(ck), B, 1001, None, 0, P(scores), None, s),          # N > max_n
        lib.fm_score(ctx, P(q), P(w), P(ck), B, N, None, 2, P(scores), None, s),             # bad mode
        lib.fm_score(ctx, P(q), P(w), P(ck_big) + 1, B, N, None, 0, P(scores), None, s),     # misaligned comp_k
        lib.fm_score(ctx, P(q) + 4, P(w), P(ck), B, N, None, 0, P(scores), None, s),         # q not 16-aligned
        lib.fm_select_topk(ctx, P(scores), B, N, None, -1, P(mask), s),                      # top_k < 0
        lib.fm_select_topk(ctx, P(scores), B, N, None, 5, None, s),                          # null mask
        lib.fm_select_threshold(ctx, P(scores), B, N, None, float("nan"), P(mask), s),       # NaN threshold
        lib.fm_select_threshold(ctx, P(scores), B, N, None, float("inf"), P(mask), s),       # inf threshold
        lib.fm_prepare_query(ctx, P(hidden), P(pos), 5, P(q), P(w), s),                      # B > max_batch
        lib.fm_prepare_query(ctx, P(hidden), None, B, P(q), P(w), s),                        # null positions
    ]
    assert cases == [EINVAL] * len(cases)
    assert L.last_error() != ""
    torch.cuda.synchronize()
    assert torch.all(scores == 7.0) and torch.all(mask == 9)


def test_success_clears_last_error(env):
    r, L = env
    L.LIB.fm_select_topk(r.ctx, None, 1, 1, None, -1, None, None)
    assert L.last_error() != ""
    s = torch.rand((1, 10), device="cuda")
    m = r.keep_topk(s, 3)
    torch.cuda.synchronize()
    assert L.last_error() == ""
    assert int(m.sum()) == 3


def test_fm_error_raised_by_binding(env):
    r, L = env
    with pytest.raises(L.FmError) as ei:
        L.fm_select_topk(r.ctx, torch.zeros((1, 2000), device="cuda"), 1, 2000, None, 1,
                         torch.zeros((1, 2000), dtype=torch.uint8, device="cuda"))
    assert ei.value.status == L.FM_EINVAL and "N = 2000" in str(ei.value)


def test_create_unsupported_and_bad_sizes(env):
    r, L = env
    out = ctypes.c_void_p()
    w = L.FmWeights()
    for i in range(3):
        w.wq_a[i] = w.q_norm[i] = w.wq_b[i] = w.w_proj[i] = r._weights[i]["wq_a"].data_ptr()
    cfg = L.config_default()
    assert L.LIB.fm_create(ctypes.byref(cfg), ctypes.byref(w), 4097, 10, ctypes.byref(out)) == L.FM_EINVAL
    assert L.LIB.fm_create(ctypes.byref(cfg), ctypes.byref(w), 4, (1 << 26) + 1, ctypes.byref(out)) == L.FM_EINVAL
    cfg.head_dim = 64
    assert L.LIB.fm_create(ctypes.byref(cfg), ctypes.byref(w), 4, 10, ctypes.byref(out)) == L.FM_EUNSUPPORTED
    assert out.value is None
    np.testing.assert_equal(L.FM_OK, 0)


def test_package_imported_before_torch_creates_a_context():
    """Importing the package before torch still gives libfm a device (the
    binding loads torch's HIP runtime first)."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import sys; sys.path.insert(0, %r); import sparse_attention_chunk_amd as fm; import synth; "
            "r = fm.FlashMemoryRetriever(fm.weights_to_device(synth.make_weights()), max_batch=1, max_n=16); "
            "r.close(); print('ok')" % root)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0 and out.stdout.strip().endswith("ok"), out.stderr[-800:]


def test_score_events_time_the_score_kernel_alone(env):
    """fm_set_score_events: the events bracket the score kernel's launch
    inside fm_score, fm_score_threshold and fm_score_fp8 (so they span less
    than the whole call), and clearing them leaves later calls alone."""
    r, L = env
    lib, ctx = L.LIB, r.ctx
    B, N = 4, 1000
    rng = np.random.default_rng(11)
    q = torch.from_numpy(rng.standard_normal((3, B, 64, 128)).astype(np.float32) * 0.1).cuda()
    w = torch.from_numpy(rng.standard_normal((3, B, 64)).astype(np.float32) * 0.01).cuda()
    ck = torch.from_numpy(rng.integers(0, 0x7f, (B, N, 132), dtype=np.uint8)).cuda()
    scores = torch.empty((B, N), device="cuda")
    mask = torch.empty((B, N), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream
    P = L.ptr
    assert lib.fm_set_score_events(ctx, None, None) == L.FM_OK
    call = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    kern = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for e in kern:
        e.record(stream)  # creates the event
    torch.cuda.synchronize()
    assert lib.fm_set_score_events(ctx, kern[0].cuda_event, None) == L.FM_EINVAL
    assert lib.fm_set_score_events(None, kern[0].cuda_event, kern[1].cuda_event) == L.FM_EINVAL
    assert lib.fm_set_score_events(ctx, kern[0].cuda_event, kern[1].cuda_event) == L.FM_OK
    try:
        calls = [
            lambda: lib.fm_score(ctx, P(q), P(w), P(ck), B, N, None, 0, P(scores), None, s),
            lambda: lib.fm_score_threshold(ctx, P(q), P(w), P(ck), B, N, None, 0, 0.5, P(scores), P(mask), None, s),
            lambda: lib.fm_score_fp8(ctx, P(q), P(w), P(ck), B, N, None, 0, P(scores), None, s),
        ]
        for c in calls:
            call[0].record(stream)
            assert c() == L.FM_OK
            call[1].record(stream)
            torch.cuda.synchronize()
            t_kern = kern[0].elapsed_time(kern[1])
            t_call = call[0].elapsed_time(call[1])
            assert 0.0 < t_kern <= t_call
    finally:
        assert lib.fm_set_score_events(ctx, None, None) == L.FM_OK
    # Ragged rows: the plan and -inf tail launch runs before the events.
    vn = torch.tensor([1000, 517, 3, 0], dtype=torch.int32, device="cuda")
    assert lib.fm_set_score_events(ctx, kern[0].cuda_event, kern[1].cuda_event) == L.FM_OK
    try:
        call[0].record(stream)
        assert lib.fm_score(ctx, P(q), P(w), P(ck), B, N, P(vn), 0, P(scores), None, s) == L.FM_OK
        call[1].record(stream)
        torch.cuda.synchronize()
        assert 0.0 < kern[0].elapsed_time(kern[1]) <= call[0].elapsed_time(call[1])
    finally:
        assert lib.fm_set_score_events(ctx, None, None) == L.FM_OK
    # Cleared: a later call records nothing, so the pair keeps its last span.
    before = kern[0].elapsed_time(kern[1])
    assert lib.fm_score(ctx, P(q), P(w), P(ck), B, N, None, 0, P(scores), None, s) == L.FM_OK
    torch.cuda.synchronize()
    assert kern[0].elapsed_time(kern[1]) == before
