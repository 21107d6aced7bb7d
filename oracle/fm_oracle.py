"""fp64 CPU oracle: query preparation, per-layer score, ensemble, selection.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Everything is float64;
fp32 inputs are promoted exactly.  No blocking, fusion or reordering beyond
what the pages' formula states: one request row at a time, one layer at a
time, numpy ``@`` for the matrix products.

Source: the FlashMemory-DeepSeek-V4 README ("FlashMemory DS-V4 Retriever"),
sections "Usage", "compressed_k format", "Architecture" and "Joint checkpoint +
ensemble", and its "Inference flow" figure for the keep-mask rule.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


# ---------------------------------------------------------------------------
# Configuration
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class OracleConfig:
    """Dimensions and constants of one indexer layer.

    README "Architecture": hidden 4096, eps 1e-6, RoPE on the last
    ROPE_DIM = 64 dims with base 160000, weight_scale = HEAD_DIM^-0.5 *
    N_HEADS^-0.5.  The hyperparameter table of the README did not survive
    extraction; N_HEADS = 64 and Q_LORA_RANK = 1024 are the stated workload's
    sizes, and HEAD_DIM = 128 follows from the record size HEAD_DIM + 4 = 132
    ("compressed_k format").  YaRN parameters: factor 1 means plain RoPE.
    """

    hidden: int = 4096
    q_lora_rank: int = 1024
    n_heads: int = 64
    head_dim: int = 128
    rope_dim: int = 64
    rms_eps: float = 1e-6
    rope_base: float = 160000.0
    yarn_factor: float = 1.0
    yarn_orig_ctx: int = 65536
    yarn_beta_fast: float = 32.0
    yarn_beta_slow: float = 1.0
    n_layers: int = 3

    @property
    def record_bytes(self) -> int:
        return self.head_dim + 4


# ---------------------------------------------------------------------------
# compressed_k decode (README "compressed_k format"; "Architecture" key branch)
# ---------------------------------------------------------------------------

def e4m3fn_value(code: int) -> float:
    """Value of one OCP FP8 E4M3 ("fn": no infinities) code.

    The pages view the first HEAD_DIM bytes as float8_e4m3.  Reading: the OCP
    e4m3fn variant (bias 7, largest finite 448, S.1111.111 is NaN).  Bits are
    S EEEE MMM; E > 0 gives (-1)^S 2^(E-7) (1 + M/8), E = 0 gives the
    subnormal (-1)^S 2^-6 (M/8).
    """
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * math.ldexp(man / 8.0, -6)
    return sign * math.ldexp(1.0 + man / 8.0, exp - 7)


def e4m3fn_table() -> np.ndarray:
    """All 256 code values, in code order, as float64."""
    return np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


_E4M3_TABLE = e4m3fn_table()


def decode_records(comp_k: np.ndarray, head_dim: int = 128) -> np.ndarray:
    """Dequantize records [..., head_dim + 4] uint8 -> k [..., head_dim] float64.

    README "compressed_k format" / "Architecture": bytes[:HEAD_DIM] viewed as
    float8_e4m3 and converted to float, times bytes[HEAD_DIM:] viewed as one
    float32 scale.  Reading: the scale is little-endian.  The product is
    exact in float64 (4-bit significand times 24-bit significand).
    """
    comp_k = np.asarray(comp_k, dtype=np.uint8)
    assert comp_k.shape[-1] == head_dim + 4
    codes = comp_k[..., :head_dim]
    scale = np.ascontiguousarray(comp_k[..., head_dim:head_dim + 4]).view("<f4")[..., 0]
    return _E4M3_TABLE[codes] * scale.astype(np.float64)[..., None]


# ---------------------------------------------------------------------------
# Query branch (README "Architecture", first diagram)
# ---------------------------------------------------------------------------

def linear(weight: np.ndarray, x: np.ndarray) -> np.ndarray:
    """y = W x for a torch-Linear-style weight [out][in], no bias.

    The pages name wq_a, wq_b and weights_proj as maps in -> out and mention
    no bias; the reading is row-major [out][in] weights and no bias.
    """
    return np.asarray(weight, dtype=np.float64) @ np.asarray(x, dtype=np.float64)


def rmsnorm(a: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm(q_norm_weight, eps) over the Q_LORA_RANK vector.

    a / sqrt(mean(a^2) + eps) * gain, eps inside the square root.
    """
    a = np.asarray(a, dtype=np.float64)
    return a / np.sqrt(np.mean(a * a) + eps) * np.asarray(gain, dtype=np.float64)


def yarn_correction_range(cfg: OracleConfig) -> tuple[float, float]:
    """Frequency-index bounds of the YaRN ramp for the rotated dims.

    The index j whose wavelength completes `r` turns over the original
    context L0 solves L0 / (2 pi base^(2j/d)) = r, i.e.
    j(r) = d ln(L0 / (2 pi r)) / (2 ln base), d = ROPE_DIM.  The fast bound
    uses r = beta_fast rounded down, the slow bound r = beta_slow rounded up,
    both clamped to [0, d - 1]; equal bounds are separated by 0.001.
    """
    d = cfg.rope_dim

    def j_of(turns: float) -> float:
        return d * math.log(cfg.yarn_orig_ctx / (turns * 2.0 * math.pi)) / (2.0 * math.log(cfg.rope_base))

    lo = max(math.floor(j_of(cfg.yarn_beta_fast)), 0)
    hi = min(math.ceil(j_of(cfg.yarn_beta_slow)), d - 1)
    lo, hi = float(lo), float(hi)
    if lo == hi:
        hi += 0.001
    return lo, hi


def rope_frequencies(cfg: OracleConfig) -> np.ndarray:
    """Per-pair angular frequencies theta'_j, j = 0 .. ROPE_DIM/2 - 1 (fp64).

    README "Architecture": RoPE (YaRN) with base 160000.  theta_j =
    base^(-2j/ROPE_DIM).  YaRN (reading: the static frequency blend, no
    attention temperature): theta'_j = theta_j (1 - ramp_j) + (theta_j / s)
    ramp_j with ramp_j = clamp((j - lo) / (hi - lo), 0, 1) over the bounds of
    `yarn_correction_range`.  s = 1 gives plain RoPE.
    """
    half = cfg.rope_dim // 2
    j = np.arange(half, dtype=np.float64)
    theta = cfg.rope_base ** (-2.0 * j / cfg.rope_dim)
    s = float(cfg.yarn_factor)
    if s == 1.0:
        return theta
    lo, hi = yarn_correction_range(cfg)
    ramp = np.clip((j - lo) / (hi - lo), 0.0, 1.0)
    return theta * (1.0 - ramp) + (theta / s) * ramp


def apply_rope(q: np.ndarray, position: int, freqs: np.ndarray, rope_dim: int) -> np.ndarray:
    """Rotate the last ROPE_DIM dims of every head vector by position * theta'.

    q: [n_heads, head_dim].  Reading: adjacent pairs (x, y) = (q[o + 2j],
    q[o + 2j + 1]), o = head_dim - rope_dim, each turned counter-clockwise by
    phi_j = position * theta'_j (angle formed in fp64):
    (x cos phi - y sin phi, x sin phi + y cos phi).  The first head_dim -
    rope_dim dims are untouched.
    """
    q = np.array(q, dtype=np.float64, copy=True)
    off = q.shape[-1] - rope_dim
    phi = float(position) * np.asarray(freqs, dtype=np.float64)
    c, s = np.cos(phi), np.sin(phi)
    x = q[..., off + 0::2].copy()
    y = q[..., off + 1::2].copy()
    q[..., off + 0::2] = x * c - y * s
    q[..., off + 1::2] = x * s + y * c
    return q


def hadamard_matrix(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix: H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]]."""
    assert n >= 1 and (n & (n - 1)) == 0
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard_transform(q: np.ndarray) -> np.ndarray:
    """Normalized Walsh-Hadamard transform of each head vector: H q / sqrt(n).

    README "Architecture": "Hadamard (normalized Walsh-Hadamard transform)",
    applied after RoPE.  Reading: Sylvester (natural) order, 1/sqrt(n).
    """
    q = np.asarray(q, dtype=np.float64)
    n = q.shape[-1]
    return q @ hadamard_matrix(n).T / math.sqrt(n)


def prepare_query_layer(layer_w: dict, hidden_row: np.ndarray, position: int, cfg: OracleConfig) -> dict:
    """One layer's query branch and weight branch for one row.

    README "Architecture": hidden -> wq_a -> RMSNorm(q_norm_weight, 1e-6) ->
    wq_b -> reshape [N_HEADS, HEAD_DIM] -> RoPE(YaRN, last 64 dims) ->
    Hadamard -> q; hidden -> weights_proj -> x HEAD_DIM^-0.5 N_HEADS^-0.5 ->
    fused_w.  Reshape reading: head-major, element (h, d) = row 128 h + d of
    the wq_b output.

    layer_w holds "wq_a" [q_lora, hidden], "q_norm" [q_lora], "wq_b"
    [n_heads * head_dim, q_lora], "w_proj" [n_heads, hidden].  Returns every
    intermediate: a, a_hat, q_lin, q_rope, q, w.
    """
    a = linear(layer_w["wq_a"], hidden_row)
    a_hat = rmsnorm(a, layer_w["q_norm"], cfg.rms_eps)
    q_lin = linear(layer_w["wq_b"], a_hat).reshape(cfg.n_heads, cfg.head_dim)
    q_rope = apply_rope(q_lin, position, rope_frequencies(cfg), cfg.rope_dim)
    q = hadamard_transform(q_rope)
    weight_scale = cfg.head_dim ** -0.5 * cfg.n_heads ** -0.5
    w = linear(layer_w["w_proj"], hidden_row) * weight_scale
    return {"a": a, "a_hat": a_hat, "q_lin": q_lin, "q_rope": q_rope, "q": q, "w": w}


def prepare_query(weights: list, hidden: np.ndarray, positions: np.ndarray, cfg: OracleConfig):
    """All layers, all rows: q [L, B, n_heads, head_dim] and w [L, B, n_heads]."""
    hidden = np.asarray(hidden, dtype=np.float64)
    positions = np.asarray(positions)
    n_rows = hidden.shape[0]
    q = np.zeros((len(weights), n_rows, cfg.n_heads, cfg.head_dim))
    w = np.zeros((len(weights), n_rows, cfg.n_heads))
    for li, lw in enumerate(weights):
        for b in range(n_rows):
            out = prepare_query_layer(lw, hidden[b], int(positions[b]), cfg)
            q[li, b] = out["q"]
            w[li, b] = out["w"]
    return q, w


# ---------------------------------------------------------------------------
# Score, ensemble, selection
# ---------------------------------------------------------------------------

def sigmoid(x: np.ndarray) -> np.ndarray:
    """Logistic function, evaluated without overflow for either sign."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def score_layer(k: np.ndarray, q: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Per-layer chunk score.

    README "Architecture": score = sigmoid(sum over heads of relu(k @ q^T) *
    fused_w), in [0, 1].  k: [N, head_dim], q: [n_heads, head_dim],
    w: [n_heads] -> [N].
    """
    logits = np.maximum(np.asarray(k, np.float64) @ np.asarray(q, np.float64).T, 0.0) @ np.asarray(w, np.float64)
    return sigmoid(logits)


def ensemble(per_layer: list, mode: str) -> np.ndarray:
    """Combine the layers' sigmoid scores per chunk.

    README "Joint checkpoint + ensemble": max (the union, the default) or
    mean across the three layers.  Reading: arithmetic mean.
    """
    stack = np.stack([np.asarray(s, np.float64) for s in per_layer])
    if mode == "max":
        return stack.max(axis=0)
    if mode == "mean":
        return stack.sum(axis=0) / stack.shape[0]
    raise ValueError(f"unknown ensemble mode {mode!r}")


def select_topk(scores: np.ndarray, valid_n: int, top_k: int) -> np.ndarray:
    """Keep mask of the top_k highest scores among the first valid_n chunks.

    README "Usage" (select_topk(top_k=512)) and "Inference flow" (keep the
    top-K chunks).  Readings: ties go to the lower chunk index; top_k above
    valid_n keeps every valid chunk; chunks at or beyond valid_n are never
    kept.
    """
    scores = np.asarray(scores, np.float64)
    n = scores.shape[0]
    valid_n = max(0, min(int(valid_n), n))
    mask = np.zeros(n, dtype=np.uint8)
    idx = np.arange(valid_n)
    order = np.lexsort((idx, -scores[:valid_n]))  # primary: score desc; secondary: index asc
    mask[order[:min(int(top_k), valid_n)]] = 1
    return mask


def select_threshold(scores: np.ndarray, valid_n: int, threshold: float) -> np.ndarray:
    """Keep mask of chunks whose score is strictly above the threshold.

    README "Usage" (select_topk(threshold=0.5)) and "Inference flow"
    ("sigmoid > thresh"): strict comparison.  Chunks at or beyond valid_n are
    never kept.
    """
    scores = np.asarray(scores, np.float64)
    n = scores.shape[0]
    valid_n = max(0, min(int(valid_n), n))
    mask = np.zeros(n, dtype=np.uint8)
    mask[:valid_n] = (scores[:valid_n] > threshold).astype(np.uint8)
    return mask


def resident_delta(mask: np.ndarray, prev_mask: np.ndarray | None = None):
    """Resident set and recall delta of one row's retrieval cycle.

    Model card "How it works": every 64 decode steps the Memory Indexer's
    selection becomes the resident_set, the chunks recalled from CPU to GPU;
    README "Inference flow": a cycle's keep mask holds for the next 64 steps.
    Returns ascending int64 index arrays (resident, entering, leaving):
    chunks kept now, kept now but not in the previous cycle (to recall), and
    kept in the previous cycle but not now (to evict).  A mask entry counts
    as kept when it is non-zero; with no previous mask every kept chunk is
    entering and none is leaving.
    """
    cur = np.asarray(mask) != 0
    prev = np.zeros_like(cur) if prev_mask is None else (np.asarray(prev_mask) != 0)
    return np.flatnonzero(cur), np.flatnonzero(cur & ~prev), np.flatnonzero(prev & ~cur)


def select_topk_subset(scores: np.ndarray, subset: np.ndarray, top_k: int) -> np.ndarray:
    """One decode step's top-K confined to the resident set, for one row.

    Model card "How it works", Level 2: the Lightning Indexer's native
    top-512 runs every step but only over the resident_set.  The pages give
    the selection, not the step's score function, so the scores are an
    input.  Readings: the subset is a list of chunk indices; entries outside
    [0, N) are never chosen; the top_k entries by score are chosen, ties
    going to the earlier list position; fewer valid entries than top_k
    chooses them all.  Returns the chosen chunk indices in list order.
    """
    scores = np.asarray(scores, np.float64)
    subset = np.asarray(subset, np.int64)
    n = scores.shape[0]
    pos = np.flatnonzero((subset >= 0) & (subset < n))
    k = min(int(top_k), len(pos))
    order = np.lexsort((pos, -scores[subset[pos]]))  # primary: score desc; secondary: position asc
    return subset[np.sort(pos[order[:k]])]


def mask_logits(logits: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """Attention logits of one request row with the dropped chunks masked.

    README "Inference flow": for the 64 decode steps after a retrieval cycle
    the attention logits of the chunks not selected are set to -inf; "What
    this simulates": such a chunk then contributes nothing to attention.
    logits [R, N] (R logit rows: heads, query positions), mask [N]; a mask
    entry keeps its chunk when it is non-zero.  Returns a new array.
    """
    out = np.array(logits, copy=True)
    out[:, np.asarray(mask) == 0] = -np.inf
    return out


def score_row(comp_k_row: np.ndarray, q_row: np.ndarray, w_row: np.ndarray, valid_n: int | None = None,
              mode: str = "max", head_dim: int = 128):
    """Scores of one request row from prepared queries.

    comp_k_row [N, head_dim + 4] uint8, q_row [L, n_heads, head_dim],
    w_row [L, n_heads].  Returns (per_layer [L, N], ensemble [N]); entries at
    or beyond valid_n are -inf (reading of the ragged-row workload: the tail
    is masked to -inf and its bytes are not read).
    """
    n = comp_k_row.shape[0]
    valid_n = n if valid_n is None else max(0, min(int(valid_n), n))
    k = decode_records(comp_k_row[:valid_n], head_dim)
    per_layer = np.full((q_row.shape[0], n), -np.inf)
    for li in range(q_row.shape[0]):
        per_layer[li, :valid_n] = score_layer(k, q_row[li], w_row[li])
    ens = np.full(n, -np.inf)
    ens[:valid_n] = ensemble([per_layer[li, :valid_n] for li in range(q_row.shape[0])], mode)
    return per_layer, ens


def run_row(weights: list, hidden_row: np.ndarray, position: int, comp_k_row: np.ndarray, cfg: OracleConfig,
            valid_n: int | None = None, mode: str = "max", top_k: int | None = None,
            threshold: float | None = None) -> dict:
    """Whole pass for one row: prepare queries, score, ensemble, select.

    README "Usage": exactly one of top_k / threshold selects the keep mask.
    """
    q = np.zeros((len(weights), cfg.n_heads, cfg.head_dim))
    w = np.zeros((len(weights), cfg.n_heads))
    for li, lw in enumerate(weights):
        out = prepare_query_layer(lw, hidden_row, position, cfg)
        q[li], w[li] = out["q"], out["w"]
    per_layer, ens = score_row(comp_k_row, q, w, valid_n, mode, cfg.head_dim)
    n = comp_k_row.shape[0]
    vn = n if valid_n is None else valid_n
    if (top_k is None) == (threshold is None):
        raise ValueError("exactly one of top_k and threshold")
    mask = select_topk(ens, vn, top_k) if top_k is not None else select_threshold(ens, vn, threshold)
    return {"q": q, "w": w, "per_layer": per_layer, "scores": ens, "mask": mask}
