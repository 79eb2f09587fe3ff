"""CPU oracle for the DSA hot path -- test infrastructure only.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package.  The product path never does.
"""
from .dsa_oracle import (  # noqa: F401
    D_VALUE, E4M3_MAX, T128_EDGES, cache_append, cache_rows, decode_bf16,
    decode_e4m3fn, decode_e8m0, decode_path, dequant_mx32, dequant_t128,
    indexer_queries, indexer_scores, indexer_scores_row, quantize_mx32, quantize_rows,
    quantize_t128, round_to_e4m3fn, sparse_mla_row, topk_row,
)
