"""The retriever interface of the FlashMemory DS-V4 README ("Usage") over libfm.

FlashMemoryRetriever wraps one libfm context built from device fp32 weights.
Calling it on (hidden, comp_k, positions) returns the three layers' scores
keyed by layer name; ensemble() combines them by max or mean; select_topk()
turns the ensemble into a boolean keep mask, either the top_k best chunks or
those above a threshold (exactly one of the two).

Also the three stages on their own (prepare_query, score, keep_topk /
keep_threshold).  Torch only allocates outputs and supplies the stream; the
arithmetic runs in libfm.
"""

from __future__ import annotations

import torch

from . import _lib

LAYER_NAMES = ("l10", "l12", "l20")
MODES = {"max": _lib.FM_ENSEMBLE_MAX, "mean": _lib.FM_ENSEMBLE_MEAN}


def _need(t, dtype, name, ndim=None):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return t


class FlashMemoryRetriever:
    """Three indexer layers (l10, l12, l20) behind one libfm context.

    weights: three dicts (l10, l12, l20) of contiguous device float32
    tensors "wq_a" [1024, 4096], "q_norm" [1024], "wq_b" [8192, 1024],
    "w_proj" [64, 4096].  They are borrowed and must outlive the object.
    yarn: optional dict with factor, orig_ctx, beta_fast, beta_slow.
    """

    def __init__(self, weights, max_batch: int = 64, max_n: int = 262144, yarn: dict | None = None,
                 rms_eps: float | None = None, rope_base: float | None = None):
        if len(weights) != 3:
            raise ValueError("three layers (l10, l12, l20) expected")
        self._weights = [{k: _need(lw[k], torch.float32, f"{k}[{i}]") for k in ("wq_a", "q_norm", "wq_b", "w_proj")}
                         for i, lw in enumerate(weights)]
        cfg = _lib.config_default()
        if yarn:
            cfg.yarn_factor = float(yarn.get("factor", 1.0))
            cfg.yarn_orig_ctx = int(yarn.get("orig_ctx", 65536))
            cfg.yarn_beta_fast = float(yarn.get("beta_fast", 32.0))
            cfg.yarn_beta_slow = float(yarn.get("beta_slow", 1.0))
        if rms_eps is not None:
            cfg.rms_eps = rms_eps
        if rope_base is not None:
            cfg.rope_base = rope_base
        w = _lib.FmWeights()
        for i, lw in enumerate(self._weights):
            w.wq_a[i] = lw["wq_a"].data_ptr()
            w.q_norm[i] = lw["q_norm"].data_ptr()
            w.wq_b[i] = lw["wq_b"].data_ptr()
            w.w_proj[i] = lw["w_proj"].data_ptr()
        self.config = cfg
        self.device = self._weights[0]["wq_a"].device
        self.max_batch, self.max_n = max_batch, max_n
        with torch.cuda.device(self.device):
            self._ctx = _lib.fm_create(cfg, w, max_batch, max_n)

    def close(self):
        if getattr(self, "_ctx", None):
            torch.cuda.synchronize(self.device)
            _lib.fm_destroy(self._ctx)
            self._ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def ctx(self) -> int:
        return self._ctx

    # ----------------------------------------------------------------- stages
    def prepare_query(self, hidden, positions):
        _need(hidden, torch.float32, "hidden", 2)
        _need(positions, torch.int64, "positions", 1)
        B = hidden.shape[0]
        q = torch.empty((3, B, 64, 128), dtype=torch.float32, device=hidden.device)
        w = torch.empty((3, B, 64), dtype=torch.float32, device=hidden.device)
        _lib.fm_prepare_query(self._ctx, hidden, positions, B, q, w)
        return q, w

    def score(self, q, w, comp_k, valid_n=None, mode="max", per_layer=False, fp8=False):
        """Per-layer and ensemble scores (fm_score); fp8=True runs the
        fp8-MFMA form (fm_score_fp8)."""
        _need(comp_k, torch.uint8, "comp_k", 3)
        _need(q, torch.float32, "q", 4)
        _need(w, torch.float32, "w", 3)
        B, N = comp_k.shape[0], comp_k.shape[1]
        if comp_k.shape[2] != 132:
            raise ValueError("comp_k records must be 132 bytes")
        if valid_n is not None:
            _need(valid_n, torch.int32, "valid_n", 1)
        scores = torch.empty((B, N), dtype=torch.float32, device=comp_k.device)
        pl = torch.empty((3, B, N), dtype=torch.float32, device=comp_k.device) if per_layer else None
        fn = _lib.fm_score_fp8 if fp8 else _lib.fm_score
        fn(self._ctx, q, w, comp_k, B, N, valid_n, MODES[mode], scores, pl)
        return (scores, pl) if per_layer else scores

    def score_select(self, q, w, comp_k, valid_n=None, mode="max", top_k=None, threshold=None, per_layer=False):
        """Scores and keep mask: fm_score + fm_select_topk, or
        fm_score_threshold (the threshold mask written by the score pass).
        Exactly one of top_k and threshold.  Returns (scores, mask) or, with
        per_layer, (scores, mask, per_layer)."""
        if (top_k is None) == (threshold is None):
            raise ValueError("pass exactly one of top_k and threshold")
        _need(comp_k, torch.uint8, "comp_k", 3)
        _need(q, torch.float32, "q", 4)
        _need(w, torch.float32, "w", 3)
        B, N = comp_k.shape[0], comp_k.shape[1]
        if comp_k.shape[2] != 132:
            raise ValueError("comp_k records must be 132 bytes")
        if valid_n is not None:
            _need(valid_n, torch.int32, "valid_n", 1)
        dev = comp_k.device
        scores = torch.empty((B, N), dtype=torch.float32, device=dev)
        mask = torch.empty((B, N), dtype=torch.bool, device=dev)
        pl = torch.empty((3, B, N), dtype=torch.float32, device=dev) if per_layer else None
        if top_k is not None:
            _lib.fm_score(self._ctx, q, w, comp_k, B, N, valid_n, MODES[mode], scores, pl)
            _lib.fm_select_topk(self._ctx, scores, B, N, valid_n, int(top_k), mask)
        else:
            _lib.fm_score_threshold(self._ctx, q, w, comp_k, B, N, valid_n, MODES[mode], float(threshold), scores,
                                    mask, pl)
        return (scores, mask, pl) if per_layer else (scores, mask)

    def keep_topk(self, scores, top_k: int, valid_n=None):
        _need(scores, torch.float32, "scores", 2)
        B, N = scores.shape
        mask = torch.empty((B, N), dtype=torch.bool, device=scores.device)
        _lib.fm_select_topk(self._ctx, scores, B, N, valid_n, int(top_k), mask)
        return mask

    def keep_threshold(self, scores, threshold: float, valid_n=None):
        _need(scores, torch.float32, "scores", 2)
        B, N = scores.shape
        mask = torch.empty((B, N), dtype=torch.bool, device=scores.device)
        _lib.fm_select_threshold(self._ctx, scores, B, N, valid_n, float(threshold), mask)
        return mask

    def resident_delta(self, mask, prev_mask=None, cap=None):
        """Resident set and recall delta of a retrieval cycle: per row the
        ascending indices of the kept chunks, of those newly kept (to recall)
        and of those no longer kept (to evict).  Returns three lists of
        int32 index tensors (one per row, length = the set's size, at most
        cap) via fm_resident_delta."""
        _need(mask, torch.bool, "mask", 2)
        B, N = mask.shape
        if prev_mask is not None:
            _need(prev_mask, torch.bool, "prev_mask", 2)
            if tuple(prev_mask.shape) != (B, N):
                raise ValueError("prev_mask shape differs from mask")
        cap = N if cap is None else int(cap)
        dev = mask.device
        lists = [torch.empty((B, max(cap, 1)), dtype=torch.int32, device=dev) for _ in range(3)]
        counts = [torch.empty((B,), dtype=torch.int32, device=dev) for _ in range(3)]
        _lib.fm_resident_delta(self._ctx, prev_mask, mask, B, N, cap, lists[0], counts[0], lists[1], counts[1],
                               lists[2], counts[2])
        n = [c.cpu() for c in counts]
        return tuple([lists[k][b, :min(int(n[k][b]), cap)] for b in range(B)] for k in range(3))

    def topk_in_subset(self, scores, subset, top_k: int, n_subset=None):
        """One decode step's top-K confined to each row's resident set
        (fm_select_topk_subset): scores [B, N] fp32 (the step's scores of
        every chunk), subset [B, cap] int32 chunk indices, n_subset [B] int32
        or None (= cap).  Returns (out [B, top_k] int32, n_out [B] int32):
        row b's chosen indices are out[b, :n_out[b]], in subset order."""
        _need(scores, torch.float32, "scores", 2)
        _need(subset, torch.int32, "subset", 2)
        B, N = scores.shape
        if subset.shape[0] != B:
            raise ValueError("subset has a different number of rows than scores")
        if n_subset is not None:
            _need(n_subset, torch.int32, "n_subset", 1)
        cap = subset.shape[1]
        out = torch.empty((B, max(int(top_k), 1)), dtype=torch.int32, device=scores.device)
        n_out = torch.empty((B,), dtype=torch.int32, device=scores.device)
        _lib.fm_select_topk_subset(self._ctx, scores, B, N, subset, n_subset, cap, int(top_k), out, n_out)
        return out[:, :int(top_k)], n_out

    def mask_logits(self, logits, mask):
        """Sets the attention logits of the chunks a keep mask drops to -inf,
        in place (fm_mask_logits).  logits [B, R, N] float32 or bfloat16,
        mask [B, N] bool.  Returns logits."""
        if logits.dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("logits must be float32 or bfloat16")
        _need(logits, logits.dtype, "logits", 3)
        _need(mask, torch.bool, "mask", 2)
        B, R, N = logits.shape
        if tuple(mask.shape) != (B, N):
            raise ValueError("mask must be [B, N] of the logits' B and N")
        dt = _lib.FM_DTYPE_F32 if logits.dtype == torch.float32 else _lib.FM_DTYPE_BF16
        _lib.fm_mask_logits(self._ctx, logits, dt, B, R, N, mask)
        return logits

    # ----------------------------------------------------- the pages' interface
    def __call__(self, hidden, comp_k, positions, valid_n=None):
        q, w = self.prepare_query(hidden, positions)
        _, pl = self.score(q, w, comp_k, valid_n, "max", per_layer=True)
        return {name: pl[i] for i, name in enumerate(LAYER_NAMES)}

    def ensemble(self, hidden, comp_k, positions, mode="max", valid_n=None):
        q, w = self.prepare_query(hidden, positions)
        return self.score(q, w, comp_k, valid_n, mode)

    def select_topk(self, hidden, comp_k, positions, top_k=None, threshold=None, mode="max", valid_n=None):
        if (top_k is None) == (threshold is None):
            raise ValueError("pass exactly one of top_k and threshold")
        q, w = self.prepare_query(hidden, positions)
        return self.score_select(q, w, comp_k, valid_n, mode, top_k=top_k, threshold=threshold)[1]


def weights_to_device(weights_np, device="cuda"):
    """Numpy fp32 layer dicts -> device tensors (contiguous)."""
    return [{k: torch.from_numpy(lw[k]).to(device).contiguous() for k in ("wq_a", "q_norm", "wq_b", "w_proj")}
            for lw in weights_np]

