"""Generator determinism and recipe checks (CPU only)."""

import hashlib
import json
import os

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _digests():
    with open(os.path.join(GOLDEN, "synth_digests.json")) as f:
        return json.load(f)


def test_unplanted_workload_digests_are_stable():
    d = _digests()
    for cid in ("1", "3", "4", "5"):
        wl = synth.WORKLOADS[int(cid)]
        assert synth.workload_inputs_digest(wl, rows=d[cid]["rows"]) == d[cid]["sha256"], cid


def test_weight_digest_is_stable():
    h = hashlib.sha256()
    for lw in synth.make_weights():
        for key in ("wq_a", "q_norm", "wq_b", "w_proj"):
            h.update(np.ascontiguousarray(lw[key]).tobytes())
    assert h.hexdigest() == _digests()["weights"]


def test_rows_are_independent_of_thread_count_and_subset():
    wl = synth.WORKLOADS[4]
    a = synth.make_comp_k(wl, rows=[3, 5], threads=1)
    b = synth.make_comp_k(wl, rows=[5], threads=1)
    c = synth.make_comp_k(wl, rows=[3, 5], threads=2)
    assert np.array_equal(a[1], b[0])
    assert np.array_equal(a, c)


def test_records_recipe():
    wl = synth.WORKLOADS[1]
    rec = synth.make_comp_k(wl)[0]
    assert rec.shape == (4096, 132) and rec.dtype == np.uint8
    codes = rec[:, :128]
    assert not np.any((codes & 0x7F) == 0x7F)                # never a NaN code
    scale = rec[:, 128:].copy().view("<f4")[:, 0]
    assert np.all(scale > 0)
    # the largest magnitude of each key is encoded as +-448 (code 0x7e / 0xfe)
    assert np.all(np.any((codes & 0x7F) == 0x7E, axis=1))


def test_ragged_tail_is_poisoned():
    wl = synth.WORKLOADS[4]
    vn = synth.make_valid_n(wl)
    assert vn.min() >= wl.n_chunks // 4 and vn.max() <= wl.n_chunks
    assert np.array_equal(synth.make_positions(wl), 4 * vn.astype(np.int64))
    rec = synth.make_comp_k(wl, rows=[0])[0]
    assert np.all(rec[vn[0]:] == 0xFF)
    assert not np.any(rec[:vn[0], :128] == 0xFF)


def test_encode_zero_key():
    rec = synth.encode_records(np.zeros((2, 128), np.float32))
    assert np.all(rec == 0)


def test_plant_plan_distinct_indices():
    wl = synth.WORKLOADS[2]
    idx, layer, head = synth.plant_plan(wl, 0)
    assert len(idx) == int(0.05 * wl.n_chunks) == len(np.unique(idx))
    assert layer.min() >= 0 and layer.max() <= 2 and head.min() >= 0 and head.max() <= 63
