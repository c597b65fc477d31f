"""CPU oracle of the QSA per-layer path -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does.
"""
from .qsa_oracle import (  # noqa: F401
    BLOCK_TOKENS,
    INDEX_DIM,
    INDEX_HEADS,
    SCORE_SCALE,
    attend,
    attend_partitioned,
    attended_tokens,
    dequantize_kv_fp8,
    dequantize_kv_q8_0,
    e4m3_decode,
    e4m3_encode,
    merge_partials,
    n_blocks,
    pool_index_keys,
    quantize_kv_fp8,
    quantize_kv_q8_0,
    qsa_row,
    score_blocks,
    select_blocks,
)
