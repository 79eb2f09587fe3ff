"""The single-kernel indexer + Top-K (dsa_indexer_topk) against the CPU
oracle: the selected positions must equal the oracle's Top-K of the oracle's
scores exactly (ties to the lower position), on the full decode batches
(bf16 and MX keys, 32 rows of 32768), on short, ragged and paged rows, rows
no longer than K, several queries per sequence, one head or one key, and
inputs with few distinct scores (long runs of ties)."""
import dataclasses

import numpy as np
import pytest
import torch

import indexed_sparse_attention_lightning_amd as dsa
import oracle
import workloads as wk
from workloads.device import to_device

from gpu_helpers import (assert_idx_equal, check_workload, paged_cache,
                         run_decode_step)

pytestmark = pytest.mark.gpu

W = wk.WORKLOADS


def oracle_idx(inp, rows, quantize=False):
    """Oracle indexer scores and Top-K of the requested rows (no attention);
    ``quantize``: the fully quantised indexer's queries."""
    wl = inp.wl
    idx = np.full((wl.B, wl.T, wl.top_k), -2, dtype=np.int64)
    for b in sorted({b for b, _ in rows}):
        keys = oracle.cache_rows(inp.k_idx.data, inp.k_idx.scale,
                                 inp.k_idx.quantized, inp.page_table[b],
                                 np.arange(inp.seq_lens[b]))
        for bb, t in rows:
            if bb != b:
                continue
            qp = int(inp.q_pos[b, t])
            n = min(qp + 1, int(inp.seq_lens[b]))
            s = oracle.indexer_scores_row(
                oracle.indexer_queries(inp.q_idx[b, t], quantize), inp.w[b, t],
                keys[:n])
            idx[b, t] = oracle.topk_row(s, qp, wl.top_k)
    return idx


def run_fused(inp, d, pass_qpos=None, q8=False):
    wl = inp.wl
    use_qpos = (wl.T > 1) if pass_qpos is None else pass_qpos
    idx = dsa.indexer_topk(paged_cache(d), d["q_idx"], d["w"], wl.top_k,
                           max_seq_len=int(inp.seq_lens.max()),
                           q_pos=d["q_pos"] if use_qpos else None,
                           quantize_queries=q8)
    torch.cuda.synchronize()
    return idx.cpu().numpy()


CASES = {
    "tiny": W["tiny"],
    # MX keys, d_I 64, 40 heads (a partial second block), ragged lengths
    # with partial last stages, scattered pages
    "paged_fp8_ragged": wk.Workload("paged_fp8_ragged", 501, B=3, T=1, H_I=40,
                                    d_I=64, top_k=300, H=16, int_range=4,
                                    quantized=True, paged_random=True,
                                    L_min=700, L_max=3000),
    # rows shorter than K (every position selected) next to longer ones
    "short_rows": wk.Workload("short_rows", 502, B=4, T=1, H_I=64, d_I=128,
                              top_k=1024, H=16, int_range=4, quantized=False,
                              paged_random=True, L_min=1, L_max=4100),
    # several queries per sequence (q_pos given), causal rows of each
    "chunk": wk.Workload("chunk", 503, B=2, T=5, H_I=16, d_I=128, top_k=256,
                         H=16, int_range=3, quantized=False, paged_random=True,
                         L=2000, first_pos=1995),
    # values in [-1, 1]: few distinct scores, long runs of equal keys
    "ties": wk.Workload("ties", 504, B=2, T=1, H_I=8, d_I=64, top_k=500,
                        H=16, int_range=1, quantized=False, paged_random=False,
                        L=6000),
    # one head, K = 1
    "one_head_k1": wk.Workload("one_head_k1", 505, B=2, T=1, H_I=1, d_I=128,
                               top_k=1, H=16, int_range=4, quantized=True,
                               paged_random=True, L=5000),
    # the longest row the fused kernel holds, MX keys, scattered pages
    "max_row_fp8": wk.Workload("max_row_fp8", 506, B=2, T=1, H_I=64, d_I=128,
                               top_k=2048, H=16, int_range=4, quantized=True,
                               paged_random=True, L=32768),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_fused_matches_oracle(name):
    wl = CASES[name]
    print(f"fused case {name}: {dataclasses.asdict(wl)}", flush=True)
    inp = wk.generate(wl)
    d = to_device(inp)
    rows = [(b, t) for b in range(wl.B) for t in range(wl.T)]
    ref = oracle_idx(inp, rows)
    assert_idx_equal(run_fused(inp, d), ref, rows)
    if wl.T == 1:   # q_pos given explicitly: the same rows
        assert_idx_equal(run_fused(inp, d, pass_qpos=True), ref, rows)


@pytest.mark.parametrize("name", ["decode", "decode_fp8"])
def test_fused_full_decode(name):
    """32 rows of 32768 positions, every row against the oracle and the
    two-kernel decode step's selection."""
    wl = W[name]
    print(f"fused full {name}", flush=True)
    inp = wk.generate(wl)
    d = to_device(inp)
    rows = [(b, 0) for b in range(wl.B)]
    got = run_fused(inp, d)
    assert_idx_equal(got, oracle_idx(inp, rows), rows)
    two, _, _ = run_decode_step(inp, d)
    assert np.array_equal(got, two)


def test_fused_repeat_is_identical():
    """Two launches give the same bytes (no state survives a launch)."""
    wl = CASES["ties"]
    inp = wk.generate(wl)
    d = to_device(inp)
    assert np.array_equal(run_fused(inp, d), run_fused(inp, d))


# 256 or more query rows with fewer than 8 queries per sequence, bf16
# queries and rows within 32768 positions: dsa_decode_step runs its indexer
# and Top-K as the single fused kernel
STEP_CASES = {
    "step_256_rows": wk.Workload("step_256_rows", 601, B=256, T=1, H_I=32,
                                 d_I=64, top_k=128, H=16, int_range=4,
                                 quantized=False, paged_random=True,
                                 L_min=60, L_max=1500),
    "step_128x2_mx": wk.Workload("step_128x2_mx", 602, B=128, T=2, H_I=64,
                                 d_I=128, top_k=256, H=16, int_range=4,
                                 quantized=True, paged_random=True, L=1200,
                                 first_pos=1198),
}


@pytest.mark.parametrize("name", sorted(STEP_CASES))
def test_decode_step_many_rows(name):
    """The whole decode step on 256 query rows: every row's indices exact and
    its attention within tolerance against the oracle, and the indices equal
    to dsa_indexer_topk's."""
    wl = STEP_CASES[name]
    print(f"decode step, fused rows {name}", flush=True)
    inp, d, _, (idx, _, _) = check_workload(wl)
    assert np.array_equal(idx, run_fused(inp, d))


def test_decode_step_many_rows_quantised():
    """The same with the fully quantised indexer (queries with fractional
    parts, MX keys): the step's fused kernel quantises the queries."""
    wl = STEP_CASES["step_128x2_mx"]
    q = wk.eighths(7004, (wl.B, wl.T, wl.H_I, wl.d_I))
    print("decode step, fused rows, quantised queries", flush=True)
    inp, d, _, (idx, _, _) = check_workload(wl, q_idx=q, quantize_queries=True)
    assert np.array_equal(idx, run_fused(inp, d, q8=True))


# The fully quantised indexer in the fused kernel: queries with fractional
# parts (multiples of 1/8, so that the MX quantisation changes them) over MX
# keys; the oracle quantises the same queries.
Q8_CASES = {
    "q8_paged_ragged": (wk.Workload("q8_paged_ragged", 701, B=3, T=1, H_I=40,
                                    d_I=64, top_k=300, H=16, int_range=4,
                                    quantized=True, paged_random=True,
                                    L_min=700, L_max=3000), 7001),
    "q8_chunk": (wk.Workload("q8_chunk", 702, B=2, T=3, H_I=64, d_I=128,
                             top_k=512, H=16, int_range=4, quantized=True,
                             paged_random=True, L=4000, first_pos=3997), 7002),
    "q8_full_decode_fp8": (W["decode_fp8"], 7003),
}


@pytest.mark.parametrize("name", sorted(Q8_CASES))
def test_fused_quantised_queries(name):
    """Every row against the oracle's quantised indexer, and (T = 1) the same
    indices as the two-kernel decode step with quantised queries."""
    wl, qseed = Q8_CASES[name]
    print(f"fused q8 case {name}", flush=True)
    inp = wk.generate(wl)
    inp = dataclasses.replace(
        inp, q_idx=wk.eighths(qseed, (wl.B, wl.T, wl.H_I, wl.d_I)))
    d = to_device(inp)
    rows = [(b, t) for b in range(wl.B) for t in range(wl.T)]
    got = run_fused(inp, d, q8=True)
    ref = oracle_idx(inp, rows, quantize=True)
    assert_idx_equal(got, ref, rows)
    plain = oracle_idx(inp, rows[:2])   # the quantisation matters here
    assert any(not np.array_equal(plain[r], ref[r]) for r in rows[:2])
    if wl.T == 1:
        two, _, _ = run_decode_step(inp, d, quantize_queries=True)
        assert np.array_equal(got, two)
