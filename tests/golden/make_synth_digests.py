"""Writes synth_digests.json: SHA-256 of generated inputs per workload.

Run from the repository root: python tests/golden/make_synth_digests.py
The planted workload's directions are the oracle's prepared queries (fp64).
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402

ROWS = {1: [0], 2: [0], 3: [0], 4: [0, 1], 5: [0]}


def plant_dirs_for(wl, rows):
    weights = synth.make_weights()
    cfg = oracle.OracleConfig()
    hidden = synth.make_hidden(wl)
    pos = synth.make_positions(wl)
    dirs = {}
    for b in rows:
        q, _ = oracle.prepare_query(weights, hidden[b:b + 1], pos[b:b + 1], cfg)
        dirs[b] = q[:, 0]
    return dirs


def main():
    out = {}
    for cid, rows in ROWS.items():
        wl = synth.WORKLOADS[cid]
        dirs = plant_dirs_for(wl, rows) if wl.plant_fraction > 0 else None
        out[str(cid)] = {"rows": rows, "sha256": synth.workload_inputs_digest(wl, rows=rows, plant_dirs=dirs)}
    w = synth.make_weights()
    import hashlib
    h = hashlib.sha256()
    for lw in w:
        for key in ("wq_a", "q_norm", "wq_b", "w_proj"):
            h.update(np.ascontiguousarray(lw[key]).tobytes())
    out["weights"] = h.hexdigest()
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "synth_digests.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(path)


if __name__ == "__main__":
    main()
