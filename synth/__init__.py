"""Seeded synthetic inputs for the Memory-Indexer scoring pass.

Shared by the tests, the smoke check and the benchmark.  It holds none of the
method's arithmetic: it draws weights, hidden states, positions, row lengths
and keys, and encodes keys into 132-byte records with torch's own float8_e4m3fn
cast.  Planted chunks (the heavy-tail workload) take their directions as an
argument; the caller supplies them.
"""

from .gen import (  # noqa: F401
    WORKLOADS,
    Workload,
    make_weights,
    make_hidden,
    make_positions,
    make_valid_n,
    plant_plan,
    encode_records,
    make_comp_k_row,
    make_comp_k,
    workload_inputs_digest,
)
