"""Oracle (test infrastructure): plain float64 CPU attention under static
block-sparse masks.  Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg may import it; the product path never
does.  It shares no code with the HIP library.  See ``attention.py``."""

from .attention import (  # noqa: F401
    ATTNSINK, BLOCKSPARSE, FULL, SLIDING, attention_backward, attention_forward,
    block_allowed, block_column, block_list_row, block_lists, blocksparse_decode_positions, decode_one, decode_positions, dense_token_mask,
    head_pattern, kv_cache_bytes, pattern_column_for_head, pattern_lists_for_head, pattern_rows_for_head,
    pattern_token_mask,
    sliding_token_mask, sparse_backward, sparse_forward, transpose_lists,
)
