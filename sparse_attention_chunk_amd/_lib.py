"""ctypes binding of libfm (include/fm.h): argument marshalling only.

Every function here has the name of the C entry point it calls and passes
raw device pointers from torch tensors plus the current HIP stream.  Every
step of the scoring pass runs in libfm's kernels; if libfm.so is missing or
fails to load, importing this module raises.
"""

from __future__ import annotations

import ctypes
import os

# torch first: libfm.so then binds to the HIP runtime torch has loaded (same
# soname), so torch's streams and device pointers are valid in libfm.  Loaded
# the other way round, the process holds two HIP runtimes and libfm's finds
# no device.
import torch  # noqa: F401

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfm.so")

FM_OK = 0
FM_EINVAL = -1
FM_EUNSUPPORTED = -2
FM_ENOMEM = -3
FM_EHIP = -4
FM_ENSEMBLE_MAX = 0
FM_ENSEMBLE_MEAN = 1
FM_DTYPE_F32 = 0
FM_DTYPE_BF16 = 1

STATUS_NAMES = {FM_OK: "FM_OK", FM_EINVAL: "FM_EINVAL", FM_EUNSUPPORTED: "FM_EUNSUPPORTED",
                FM_ENOMEM: "FM_ENOMEM", FM_EHIP: "FM_EHIP"}

# Exported symbols, in header order.
EXPORTS = ("fm_config_default", "fm_create", "fm_destroy", "fm_prepare_query", "fm_score", "fm_score_threshold",
           "fm_score_fp8", "fm_select_topk", "fm_select_topk_static", "fm_select_topk_subset", "fm_select_threshold", "fm_resident_delta",
           "fm_mask_logits", "fm_set_score_events", "fm_last_error")


class FmConfig(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("q_lora_rank", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("rope_dim", ctypes.c_int32),
        ("rms_eps", ctypes.c_float),
        ("rope_base", ctypes.c_double),
        ("yarn_factor", ctypes.c_double),
        ("yarn_orig_ctx", ctypes.c_int64),
        ("yarn_beta_fast", ctypes.c_double),
        ("yarn_beta_slow", ctypes.c_double),
    ]


class FmWeights(ctypes.Structure):
    _fields_ = [
        ("wq_a", ctypes.c_void_p * 3),
        ("q_norm", ctypes.c_void_p * 3),
        ("wq_b", ctypes.c_void_p * 3),
        ("w_proj", ctypes.c_void_p * 3),
    ]


class FmError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libfm.so is not built at {LIB_PATH}: run `python sparse_attention_chunk_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.fm_config_default.argtypes = [ctypes.POINTER(FmConfig)]
    lib.fm_config_default.restype = None
    lib.fm_create.argtypes = [ctypes.POINTER(FmConfig), ctypes.POINTER(FmWeights), i32, i64, ctypes.POINTER(vp)]
    lib.fm_create.restype = ctypes.c_int
    lib.fm_destroy.argtypes = [vp]
    lib.fm_destroy.restype = None
    lib.fm_prepare_query.argtypes = [vp, vp, vp, i32, vp, vp, vp]
    lib.fm_prepare_query.restype = ctypes.c_int
    lib.fm_score.argtypes = [vp, vp, vp, vp, i32, i64, vp, ctypes.c_int, vp, vp, vp]
    lib.fm_score.restype = ctypes.c_int
    lib.fm_score_threshold.argtypes = [vp, vp, vp, vp, i32, i64, vp, ctypes.c_int, ctypes.c_float, vp, vp, vp, vp]
    lib.fm_score_threshold.restype = ctypes.c_int
    lib.fm_score_fp8.argtypes = [vp, vp, vp, vp, i32, i64, vp, ctypes.c_int, vp, vp, vp]
    lib.fm_score_fp8.restype = ctypes.c_int
    lib.fm_select_topk.argtypes = [vp, vp, i32, i64, vp, i32, vp, vp]
    lib.fm_select_topk.restype = ctypes.c_int
    lib.fm_select_topk_static.argtypes = [vp, i32, i64, vp, i32, vp, vp]
    lib.fm_select_topk_static.restype = ctypes.c_int
    lib.fm_select_topk_subset.argtypes = [vp, vp, i32, i64, vp, vp, i32, i32, vp, vp, vp]
    lib.fm_select_topk_subset.restype = ctypes.c_int
    lib.fm_select_threshold.argtypes = [vp, vp, i32, i64, vp, ctypes.c_float, vp, vp]
    lib.fm_select_threshold.restype = ctypes.c_int
    lib.fm_mask_logits.argtypes = [vp, vp, ctypes.c_int, i32, i32, i64, vp, vp]
    lib.fm_mask_logits.restype = ctypes.c_int
    lib.fm_resident_delta.argtypes = [vp, vp, vp, i32, i64, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.fm_resident_delta.restype = ctypes.c_int
    lib.fm_set_score_events.argtypes = [vp, vp, vp]
    lib.fm_set_score_events.restype = ctypes.c_int
    lib.fm_last_error.argtypes = []
    lib.fm_last_error.restype = ctypes.c_char_p
    return lib


LIB = _load()


def last_error() -> str:
    return LIB.fm_last_error().decode()


def check(status: int, where: str) -> None:
    if status != FM_OK:
        raise FmError(status, where, last_error())


def ptr(t) -> int | None:
    """Device address of a tensor (None passes NULL)."""
    return None if t is None else t.data_ptr()


def current_stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def config_default() -> FmConfig:
    cfg = FmConfig()
    LIB.fm_config_default(ctypes.byref(cfg))
    return cfg


def fm_create(cfg: FmConfig, weights: FmWeights, max_batch: int, max_n: int) -> int:
    out = ctypes.c_void_p()
    check(LIB.fm_create(ctypes.byref(cfg), ctypes.byref(weights), max_batch, max_n, ctypes.byref(out)), "fm_create")
    return out.value


def fm_destroy(ctx: int) -> None:
    LIB.fm_destroy(ctx)


def fm_prepare_query(ctx, hidden, positions, B, q_out, w_out, stream=None) -> None:
    s = current_stream() if stream is None else stream
    check(LIB.fm_prepare_query(ctx, ptr(hidden), ptr(positions), B, ptr(q_out), ptr(w_out), s), "fm_prepare_query")


def fm_score(ctx, q, w, comp_k, B, N, valid_n, mode, scores, per_layer=None, stream=None) -> None:
    s = current_stream() if stream is None else stream
    check(LIB.fm_score(ctx, ptr(q), ptr(w), ptr(comp_k), B, N, ptr(valid_n), mode, ptr(scores), ptr(per_layer), s),
          "fm_score")


def fm_score_threshold(ctx, q, w, comp_k, B, N, valid_n, mode, threshold, scores, mask, per_layer=None,
                       stream=None) -> None:
    s = current_stream() if stream is None else stream
    check(LIB.fm_score_threshold(ctx, ptr(q), ptr(w), ptr(comp_k), B, N, ptr(valid_n), mode, threshold, ptr(scores),
                                 ptr(mask), ptr(per_layer), s), "fm_score_threshold")


def fm_score_fp8(ctx, q, w, comp_k, B, N, valid_n, mode, scores, per_layer=None, stream=None) -> None:
    s = current_stream() if stream is None else stream
    check(LIB.fm_score_fp8(ctx, ptr(q), ptr(w), ptr(comp_k), B, N, ptr(valid_n), mode, ptr(scores), ptr(per_layer),
                           s), "fm_score_fp8")


def fm_select_topk(ctx, scores, B, N, valid_n, top_k, mask, stream=None) -> None:
    s = current_stream() if stream is None else stream
    check(LIB.fm_select_topk(ctx, ptr(scores), B, N, ptr(valid_n), top_k, ptr(mask), s), "fm_select_topk")


def fm_select_topk_static(scores, B, N, valid_n, top_k, mask, stream=None) -> None:
    s = current_stream() if stream is None else stream
    check(LIB.fm_select_topk_static(ptr(scores), B, N, ptr(valid_n), top_k, ptr(mask), s), "fm_select_topk_static")


def fm_select_topk_subset(ctx, scores, B, N, subset, n_subset, cap, top_k, out, n_out, stream=None) -> None:
    s = current_stream() if stream is None else stream
    check(LIB.fm_select_topk_subset(ctx, ptr(scores), B, N, ptr(subset), ptr(n_subset), cap, top_k, ptr(out),
                                    ptr(n_out), s), "fm_select_topk_subset")


def fm_select_threshold(ctx, scores, B, N, valid_n, threshold, mask, stream=None) -> None:
    s = current_stream() if stream is None else stream
    check(LIB.fm_select_threshold(ctx, ptr(scores), B, N, ptr(valid_n), threshold, ptr(mask), s),
          "fm_select_threshold")


def fm_mask_logits(ctx, logits, dtype, B, R, N, mask, stream=None) -> None:
    s = current_stream() if stream is None else stream
    check(LIB.fm_mask_logits(ctx, ptr(logits), dtype, B, R, N, ptr(mask), s), "fm_mask_logits")


def fm_set_score_events(ctx, before, after) -> None:
    """before/after: hipEvent_t handles (ints or ctypes.c_void_p), or both None."""
    check(LIB.fm_set_score_events(ctx, before, after), "fm_set_score_events")


def fm_resident_delta(ctx, prev_mask, mask, B, N, cap, resident, n_resident, entering=None, n_entering=None,
                      leaving=None, n_leaving=None, stream=None) -> None:
    s = current_stream() if stream is None else stream
    check(LIB.fm_resident_delta(ctx, ptr(prev_mask), ptr(mask), B, N, cap, ptr(resident), ptr(n_resident),
                                ptr(entering), ptr(n_entering), ptr(leaving), ptr(n_leaving), s),
          "fm_resident_delta")
