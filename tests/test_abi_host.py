"""The C ABI library loads and exports what include/fm.h declares (CPU only:
no call here reaches the GPU; every call checks its arguments before any
HIP runtime call)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fm.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fm_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert _declared() == sorted(["fm_config_default", "fm_create", "fm_destroy", "fm_prepare_query", "fm_score",
                                  "fm_score_threshold", "fm_score_fp8",
                                  "fm_select_topk", "fm_select_topk_static", "fm_select_topk_subset",
                                  "fm_select_threshold",
                                  "fm_mask_logits", "fm_resident_delta", "fm_set_score_events",
                                  "fm_last_error"])


def test_library_exports_every_declared_symbol():
    from sparse_attention_chunk_amd import _lib
    for name in _declared():
        assert hasattr(_lib.LIB, name), name
        assert ctypes.cast(getattr(_lib.LIB, name), ctypes.c_void_p).value
    assert set(_lib.EXPORTS) == set(_declared())


def test_config_default_values():
    from sparse_attention_chunk_amd import _lib
    c = _lib.config_default()
    assert (c.n_layers, c.hidden, c.q_lora_rank, c.n_heads, c.head_dim, c.rope_dim) == (3, 4096, 1024, 64, 128, 64)
    assert c.rms_eps == pytest.approx(1e-6) and c.rope_base == 160000.0 and c.yarn_factor == 1.0
    assert (c.yarn_orig_ctx, c.yarn_beta_fast, c.yarn_beta_slow) == (65536, 32.0, 1.0)


def test_struct_layout_matches_header():
    from sparse_attention_chunk_amd import _lib
    # int32 x6, float, (pad), double, double, int64, double, double
    assert ctypes.sizeof(_lib.FmConfig) == 6 * 4 + 4 + 4 + 5 * 8
    assert ctypes.sizeof(_lib.FmWeights) == 12 * ctypes.sizeof(ctypes.c_void_p)


def test_null_context_is_rejected_before_any_launch():
    from sparse_attention_chunk_amd import _lib
    L = _lib.LIB
    assert L.fm_prepare_query(None, None, None, 1, None, None, None) == _lib.FM_EINVAL
    assert "null context" in _lib.last_error()
    assert L.fm_score(None, None, None, None, 1, 1, None, 0, None, None, None) == _lib.FM_EINVAL
    assert L.fm_score_fp8(None, None, None, None, 1, 1, None, 0, None, None, None) == _lib.FM_EINVAL
    assert L.fm_score_threshold(None, None, None, None, 1, 1, None, 0, 0.5, None, None, None, None) == _lib.FM_EINVAL
    assert L.fm_select_topk(None, None, 1, 1, None, 1, None, None) == _lib.FM_EINVAL
    assert L.fm_select_threshold(None, None, 1, 1, None, 0.5, None, None) == _lib.FM_EINVAL
    assert L.fm_select_topk_subset(None, None, 1, 1, None, None, 1, 1, None, None, None) == _lib.FM_EINVAL
    assert L.fm_mask_logits(None, None, 0, 1, 1, 1, None, None) == _lib.FM_EINVAL
    assert L.fm_set_score_events(None, None, None) == _lib.FM_EINVAL
    L.fm_destroy(None)  # no-op


def test_static_topk_rejects_sizes_beyond_its_scratch_before_touching_the_device():
    from sparse_attention_chunk_amd import _lib
    L = _lib.LIB
    assert L.fm_select_topk_static(None, 70000, 16, None, 1, None, None) == _lib.FM_EINVAL
    assert "65535" in _lib.last_error()
    assert L.fm_select_topk_static(None, 1, (1 << 26) + 1, None, 1, None, None) == _lib.FM_EINVAL
    # 8 bytes per 16 chunks (rounded up to an even count) of each row: B = 64, N = 262144 needs 8 MiB exactly
    assert L.fm_select_topk_static(None, 65, 262144, None, 512, None, None) == _lib.FM_EINVAL
    assert "static scratch" in _lib.last_error()
    assert L.fm_select_topk_static(None, 64, 262144, None, 512, None, None) == _lib.FM_EINVAL
    assert "null pointer" in _lib.last_error()
    assert L.fm_select_topk_static(None, 1, 16, None, -1, None, None) == _lib.FM_EINVAL
    assert L.fm_select_topk_static(None, 0, 16, None, 1, None, None) == _lib.FM_OK


def test_create_rejects_bad_config_before_touching_the_device():
    from sparse_attention_chunk_amd import _lib
    out = ctypes.c_void_p()
    w = _lib.FmWeights()
    cfg = _lib.config_default()
    cfg.n_heads = 32
    assert _lib.LIB.fm_create(ctypes.byref(cfg), ctypes.byref(w), 8, 1024, ctypes.byref(out)) == _lib.FM_EUNSUPPORTED
    cfg = _lib.config_default()
    cfg.yarn_factor = 0.5
    assert _lib.LIB.fm_create(ctypes.byref(cfg), ctypes.byref(w), 8, 1024, ctypes.byref(out)) == _lib.FM_EINVAL
    cfg = _lib.config_default()
    assert _lib.LIB.fm_create(ctypes.byref(cfg), ctypes.byref(w), 0, 1024, ctypes.byref(out)) == _lib.FM_EINVAL
    assert _lib.LIB.fm_create(ctypes.byref(cfg), ctypes.byref(w), 8, 1024, ctypes.byref(out)) == _lib.FM_EINVAL  # null weights
    assert "null weight" in _lib.last_error()
    assert _lib.LIB.fm_create(None, ctypes.byref(w), 8, 1024, ctypes.byref(out)) == _lib.FM_EINVAL
    assert out.value is None


def test_binding_loads_torch_before_libfm():
    """libfm.so must bind to torch's HIP runtime: the binding imports torch
    before it loads the library (checked in a fresh interpreter)."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r); import sparse_attention_chunk_amd._lib as L; "
            "import sys as s; print('torch' in s.modules)" % ROOT)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr[-500:]
    assert out.stdout.strip().endswith("True")


def test_plain_c_caller_builds_and_runs(tmp_path):
    """include/fm.h compiles as strict C99 and a C program linked against
    libfm.so gets the defaults and the host-side argument checks
    (tests/abi_c/abi_check.c)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    pkg = os.path.join(ROOT, "sparse_attention_chunk_amd")
    if not os.path.exists(os.path.join(pkg, "libfm.so")):
        pytest.skip("libfm.so is not built")
    exe = str(tmp_path / "abi_check")
    build = subprocess.run([gcc, "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
                            "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "abi_c", "abi_check.c"),
                            "-L", pkg, "-l:libfm.so", "-Wl,-rpath," + pkg, "-o", exe],
                           capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
    assert run.stdout.strip() == "ok"
