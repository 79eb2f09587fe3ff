"""CPU oracle for the DSA hot path -- test infrastructure only.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package.  The product path never does.
"""
from .dsa_oracle import (  # noqa: F401
    D_VALUE, cache_rows, decode_bf16, decode_e4m3fn, decode_e8m0,
    decode_path, dequant_mx32, indexer_scores, indexer_scores_row,
    sparse_mla_row, topk_row,
)
