"""CPU oracle (test infrastructure only; see indexcache_oracle)."""
from .indexcache_oracle import (  # noqa: F401
    NoCachedIndices,
    decode,
    decode_bf16,
    decode_e4m3,
    decode_step,
    indexer_scores,
    indexer_scores_row,
    indexer_topk,
    is_full,
    jaccard_rows,
    run_stack,
    sparse_attn,
    sparse_attn_row,
    to_decision_precision,
    topk_row,
)
