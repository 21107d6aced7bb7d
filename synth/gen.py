"""Seeded generators (numpy PCG64 streams keyed by SeedSequence).

Stream keys:
  weights of layer l (0, 1, 2 = l10, l12, l20), tensor t (0 wq_a, 1 q_norm,
  2 wq_b, 3 w_proj): [0, l, t]
  workload c: hidden [c, 1], positions [c, 2], valid_n [c, 3],
  keys of row b [c, 100, b], planting plan of row b [c, 200, b].

"N(0, v)" below means variance v.  Weights are drawn as float64 normals,
scaled and cast to float32; keys are drawn directly as float32 normals (the
bulk of the bytes), one independent stream per row so that any row subset
can be regenerated on its own.
"""

from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
from dataclasses import dataclass, field

import numpy as np
import torch

RECORD_BYTES = 132
HEAD_DIM = 128
FP8_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, position rule, ensemble and selection."""

    cid: int
    name: str
    batch: int
    n_chunks: int
    mode: str = "max"
    top_k: int | None = 512
    threshold: float | None = None
    yarn_factor: float = 1.0
    yarn_orig_ctx: int = 65536
    yarn_beta_fast: float = 32.0
    yarn_beta_slow: float = 1.0
    ragged: bool = False
    plant_fraction: float = 0.0
    position_rule: str = "4n"          # "fixed", "4n", "uniform", "4valid"
    position_fixed: int = 0
    position_range: tuple = (0, 0)
    extra_selects: tuple = field(default=())  # additional (mode, top_k, threshold) runs on the same inputs


WORKLOADS = {
    1: Workload(1, "b1_n4096_max_top512", 1, 4096, position_rule="fixed", position_fixed=16384),
    2: Workload(2, "b8_n65536_planted5pct_max_top512", 8, 65536, plant_fraction=0.05),
    3: Workload(3, "b32_n131072_mean_thr0.5", 32, 131072, mode="mean", top_k=None, threshold=0.5,
                position_rule="uniform", position_range=(262144, 524288)),
    4: Workload(4, "b60_n131072_ragged_yarn4_max_top1024", 60, 131072, top_k=1024, yarn_factor=4.0,
                ragged=True, position_rule="4valid"),
    5: Workload(5, "b30_n262144_max_top512", 30, 262144,
                extra_selects=(("mean", 512, None), ("max", None, 0.5))),
}


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def make_weights(n_layers: int = 3, hidden: int = 4096, q_lora_rank: int = 1024, n_heads: int = 64,
                 head_dim: int = 128) -> list:
    """Random-init indexer weights, float32, torch-Linear layout [out][in].

    wq_a ~ N(0, 1/hidden), q_norm = 1 + N(0, 0.02), wq_b ~ N(0, 1/q_lora_rank),
    w_proj ~ N(0, 1/hidden).
    """
    layers = []
    for li in range(n_layers):
        wq_a = _rng(0, li, 0).standard_normal((q_lora_rank, hidden)) * (1.0 / hidden) ** 0.5
        q_norm = 1.0 + _rng(0, li, 1).standard_normal(q_lora_rank) * 0.02 ** 0.5
        wq_b = _rng(0, li, 2).standard_normal((n_heads * head_dim, q_lora_rank)) * (1.0 / q_lora_rank) ** 0.5
        w_proj = _rng(0, li, 3).standard_normal((n_heads, hidden)) * (1.0 / hidden) ** 0.5
        layers.append({
            "wq_a": wq_a.astype(np.float32),
            "q_norm": q_norm.astype(np.float32),
            "wq_b": wq_b.astype(np.float32),
            "w_proj": w_proj.astype(np.float32),
        })
    return layers


def make_hidden(wl: Workload, hidden: int = 4096) -> np.ndarray:
    """Decode-token hidden states [B, hidden] ~ N(0, 1), float32."""
    return _rng(wl.cid, 1).standard_normal((wl.batch, hidden)).astype(np.float32)


def make_valid_n(wl: Workload) -> np.ndarray:
    """Valid chunks per row, int32: N for every row unless the workload is
    ragged, then uniform on [N/4, N] inclusive."""
    if not wl.ragged:
        return np.full(wl.batch, wl.n_chunks, dtype=np.int32)
    lo = wl.n_chunks // 4
    return _rng(wl.cid, 3).integers(lo, wl.n_chunks + 1, size=wl.batch).astype(np.int32)


def make_positions(wl: Workload) -> np.ndarray:
    """Token positions [B] int64.  The decode token follows a context at 4x
    compression (position = 4 * chunks) unless the workload fixes it."""
    if wl.position_rule == "fixed":
        return np.full(wl.batch, wl.position_fixed, dtype=np.int64)
    if wl.position_rule == "4n":
        return np.full(wl.batch, 4 * wl.n_chunks, dtype=np.int64)
    if wl.position_rule == "4valid":
        return 4 * make_valid_n(wl).astype(np.int64)
    if wl.position_rule == "uniform":
        lo, hi = wl.position_range
        return _rng(wl.cid, 2).integers(lo, hi, size=wl.batch).astype(np.int64)
    raise ValueError(wl.position_rule)


def plant_plan(wl: Workload, b: int, n_layers: int = 3, n_heads: int = 64):
    """Planted chunks of row b: (indices, layer, head), floor(f N) distinct
    chunk indices drawn without replacement, each with a uniform layer/head."""
    n_plant = int(np.floor(wl.plant_fraction * wl.n_chunks))
    if n_plant == 0:
        return np.zeros(0, np.int64), np.zeros(0, np.int64), np.zeros(0, np.int64)
    rng = _rng(wl.cid, 200, b)
    idx = rng.choice(wl.n_chunks, size=n_plant, replace=False).astype(np.int64)
    layer = rng.integers(0, n_layers, size=n_plant).astype(np.int64)
    head = rng.integers(0, n_heads, size=n_plant).astype(np.int64)
    return idx, layer, head


def encode_records(keys: np.ndarray) -> np.ndarray:
    """Encode float32 keys [n, 128] into records [n, 132] uint8.

    scale = absmax / 448 in float32 (0 for an all-zero key), codes = the
    float8_e4m3fn cast (torch, round to nearest even) of key / scale clamped
    to +-448, so no NaN code is ever produced; the scale follows the codes
    as a little-endian float32.
    """
    kt = torch.from_numpy(np.ascontiguousarray(keys, dtype=np.float32))
    n = kt.shape[0]
    scale = kt.abs().amax(dim=1) / FP8_MAX
    zero = scale == 0
    safe = torch.where(zero, torch.ones_like(scale), scale)
    x = (kt / safe[:, None]).clamp_(-FP8_MAX, FP8_MAX)
    codes = x.to(torch.float8_e4m3fn).view(torch.uint8)
    codes[zero] = 0
    out = np.empty((n, RECORD_BYTES), dtype=np.uint8)
    out[:, :HEAD_DIM] = codes.numpy()
    out[:, HEAD_DIM:] = scale.numpy().astype("<f4").view(np.uint8).reshape(n, 4)
    return out


def make_comp_k_row(wl: Workload, b: int, plant_dirs: np.ndarray | None = None,
                    out: np.ndarray | None = None) -> np.ndarray:
    """Records of row b: [N, 132] uint8.

    Keys ~ N(0, 1)^128 per chunk.  Planted chunks (plant_fraction > 0) take
    the key 0.5 * plant_dirs[layer, head] instead; plant_dirs [3, 64, 128] is
    the row's prepared query, supplied by the caller.  Chunks at or beyond
    the row's valid length are filled with 0xFF bytes (NaN codes and a NaN
    scale): they must never be read.
    """
    n = wl.n_chunks
    if out is None:
        out = np.empty((n, RECORD_BYTES), dtype=np.uint8)
    valid = int(make_valid_n(wl)[b])
    keys = _rng(wl.cid, 100, b).standard_normal((n, HEAD_DIM), dtype=np.float32)
    if wl.plant_fraction > 0:
        if plant_dirs is None:
            raise ValueError("this workload plants keys along the row's queries: pass plant_dirs")
        idx, layer, head = plant_plan(wl, b, plant_dirs.shape[0], plant_dirs.shape[1])
        keys[idx] = (0.5 * np.asarray(plant_dirs, np.float64)[layer, head]).astype(np.float32)
    out[:valid] = encode_records(keys[:valid])
    out[valid:] = 0xFF
    return out


def make_comp_k(wl: Workload, rows=None, plant_dirs=None, threads: int | None = None) -> np.ndarray:
    """Records for a set of rows (default: all), [len(rows), N, 132] uint8.

    plant_dirs, when the workload plants, is indexable by row: plant_dirs[b]
    is [3, 64, 128].  Rows are generated in parallel threads; each row has
    its own stream, so the result does not depend on the thread count.
    """
    rows = list(range(wl.batch)) if rows is None else list(rows)
    out = np.empty((len(rows), wl.n_chunks, RECORD_BYTES), dtype=np.uint8)
    if threads is None:
        threads = max(1, min(len(rows), len(os.sched_getaffinity(0)), 16))

    def one(i):
        b = rows[i]
        make_comp_k_row(wl, b, None if plant_dirs is None else plant_dirs[b], out=out[i])

    if threads == 1 or len(rows) == 1:
        for i in range(len(rows)):
            one(i)
    else:
        prev = torch.get_num_threads()
        torch.set_num_threads(1)
        try:
            with cf.ThreadPoolExecutor(threads) as ex:
                list(ex.map(one, range(len(rows))))
        finally:
            torch.set_num_threads(prev)
    return out


def workload_inputs_digest(wl: Workload, rows=None, plant_dirs=None) -> str:
    """SHA-256 over hidden, positions, valid_n and the records of `rows`."""
    h = hashlib.sha256()
    h.update(make_hidden(wl).tobytes())
    h.update(make_positions(wl).tobytes())
    h.update(make_valid_n(wl).tobytes())
    h.update(make_comp_k(wl, rows=rows, plant_dirs=plant_dirs).tobytes())
    return h.hexdigest()
