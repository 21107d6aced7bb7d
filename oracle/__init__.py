"""Plain fp64 CPU oracle for the FlashMemory Memory-Indexer scoring pass.

TEST INFRASTRUCTURE ONLY.  This package is the checker that the HIP library is
measured against.  Only the test suite, the smoke check in ``__graft_entry__``
and the ``cpu_baseline`` leg of ``bench.py`` may import it; the product path
(``sparse_attention_chunk_amd``) never does, and it shares no code, table or
constant with that path.

Every function cites the passage of the FlashMemory-DeepSeek-V4 pages it
follows ("FlashMemory DS-V4 Retriever" README, section "Architecture", its
"compressed_k format" section, and the "Joint checkpoint + ensemble" and
"Inference flow" sections).  Where the pages are silent the plain reading
taken is named in the function's docstring.

Pins (what fixes each function independently of this code) live in
``tests/test_oracle_pins.py``.  The one function without an independent pin
is the composed pipeline on real trained data: parity unpinned there, since
the pages ship no weights, keys or worked example.
"""

from .fm_oracle import (  # noqa: F401
    OracleConfig,
    e4m3fn_value,
    e4m3fn_table,
    decode_records,
    linear,
    rmsnorm,
    rope_frequencies,
    yarn_correction_range,
    apply_rope,
    hadamard_matrix,
    hadamard_transform,
    prepare_query_layer,
    prepare_query,
    sigmoid,
    score_layer,
    ensemble,
    select_topk,
    select_threshold,
    select_topk_subset,
    resident_delta,
    mask_logits,
    score_row,
    run_row,
)
