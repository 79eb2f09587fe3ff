"""The fully quantised indexer (queries quantised to MX block-32 on the fly,
scaled FP8 matrix cores over MX keys) vs the CPU oracle with the same query
quantisation (needs an MI355X).

Queries are multiples of 1/8 (about a third of them change under the
quantisation) and keys small integers, so every score is exact in fp32:
scores must match bit for bit, indices exactly, attention within the usual
tolerances.
"""
import numpy as np
import pytest

import oracle
import workloads as wk

from gpu_helpers import check_workload, prefill_rows

pytestmark = pytest.mark.gpu

W = wk.WORKLOADS

Q8_CASES = {
    "decode_fp8": wk.scaled(W["decode_fp8"], B=3, L=2048, top_k=256, seed=121),
    "decode_fp8_unaligned": wk.scaled(W["decode_fp8"], B=2, L=1000,
                                      top_k=300, seed=122),
    "paged_fp8": wk.scaled(W["ragged"], B=3, L_min=100, L_max=3000,
                           top_k=512, seed=123),
    "paged_small_heads": wk.scaled(W["ragged"], B=2, L_min=700, L_max=1300,
                                   top_k=128, H=40, H_I=20, d_I=64, seed=124),
    "prefill_fp8": wk.scaled(W["prefill"], T=37, L=1000, first_pos=900,
                             top_k=300, H=32, quantized=True, seed=125),
    "prefill_small_dims": wk.scaled(W["prefill"], T=19, L=700, first_pos=600,
                                    top_k=128, H=16, H_I=20, d_I=64,
                                    quantized=True, seed=126),
}


@pytest.mark.parametrize("name", sorted(Q8_CASES))
def test_quantised_indexer_matches_oracle(name):
    wl = Q8_CASES[name]
    q = wk.eighths(wl.seed + 1000, (wl.B, wl.T, wl.H_I, wl.d_I))
    print(f"q8 case {name}", flush=True)
    inp, d, ref, _ = check_workload(wl, q_idx=q, quantize_queries=True)
    # the quantised path really differs from the bf16-query one here
    rows = [(b, t) for b in range(wl.B) for t in range(wl.T)][:4]
    plain = oracle.decode_path(inp, rows=rows, want_scores=True)
    assert any(not np.array_equal(plain["scores"][r], ref["scores"][r])
               for r in rows)


def test_quantised_indexer_full_decode_fp8():
    """The FP8 decode batch at full size (32 x 32768), every row."""
    wl = W["decode_fp8"]
    q = wk.eighths(1001, (wl.B, wl.T, wl.H_I, wl.d_I))
    print("q8 full decode_fp8", flush=True)
    check_workload(wl, q_idx=q, quantize_queries=True)


def test_quantised_indexer_full_prefill_chunk():
    """The 4096-query prefill chunk over a 65536-token MX cache, sampled
    rows (the query-tiled quantised kernel at full size)."""
    wl = wk.scaled(W["prefill"], quantized=True)
    q = wk.eighths(1002, (wl.B, wl.T, wl.H_I, wl.d_I))
    print("q8 full prefill chunk", flush=True)
    check_workload(wl, rows=prefill_rows(), q_idx=q, quantize_queries=True)
