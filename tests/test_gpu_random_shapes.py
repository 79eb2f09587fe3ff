"""Seeded random shapes through the whole decode step (and the separate
entry points where the cache is contiguous), HIP path vs CPU oracle.

Each case draws, from its own fixed seed, a batch, query count, head
counts, indexer width, top_k, context length and storage formats within
the C ABI's support set: lengths below one key stage or one attention tile,
top_k larger than the history, single heads, prefill chunks that start at
position 0 or run to the end of the context, scattered pages, MX keys and
KV, and the fully quantised indexer.  The bars are those of the other
parity tests (exact Top-K sets and scores, attention within its tolerance).
Cases with bf16 indexer queries also run the single-kernel indexer + Top-K
(dsa_indexer_topk), whose indices must equal the oracle's.
"""
import dataclasses

import numpy as np
import pytest
import torch

import indexed_sparse_attention_lightning_amd as dsa
import workloads as wk

from gpu_helpers import assert_idx_equal, check_workload, paged_cache

pytestmark = pytest.mark.gpu

N_CASES = 48


def draw_case(i):
    """Workload and the quantised-indexer flag of case i (fixed seed)."""
    rng = np.random.default_rng(9100 + i)
    kind = ("decode", "ragged", "prefill")[i % 3]
    quantized = bool(rng.integers(0, 2))
    d_I = int(rng.choice([64, 128]))
    H_I = int(rng.integers(1, 65))
    H = int(rng.integers(1, 129))
    top_k = int(rng.choice([1, int(rng.integers(2, 300)), int(rng.integers(300, 2049))]))
    base = dict(name=f"random_{i}", seed=9200 + i, H_I=H_I, d_I=d_I, top_k=top_k,
                H=H, int_range=int(rng.integers(1, 5)), quantized=quantized)
    if kind == "decode":
        L = int(rng.choice([int(rng.integers(1, 33)), int(rng.integers(33, 3000))]))
        wl = wk.Workload(B=int(rng.integers(1, 5)), T=1, L=L,
                         paged_random=bool(rng.integers(0, 2)), **base)
    elif kind == "ragged":
        lo = int(rng.integers(1, 1500))
        wl = wk.Workload(B=int(rng.integers(1, 5)), T=1, L_min=lo,
                         L_max=lo + int(rng.integers(0, 2500)),
                         paged_random=True, **base)
    else:
        L = int(rng.integers(16, 2500))
        T = int(rng.integers(2, min(L, 48) + 1))
        first = int(rng.choice([0, L - T, int(rng.integers(0, L - T + 1))]))
        wl = wk.Workload(B=int(rng.integers(1, 3)), T=T, L=L, first_pos=first,
                         paged_random=bool(rng.integers(0, 2)), **base)
    q8 = quantized and bool(rng.integers(0, 2))
    return wl, q8


CASES = [draw_case(i) for i in range(N_CASES)]


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shapes(i):
    wl, q8 = CASES[i]
    print(f"case {i}: {dataclasses.asdict(wl)} q8={q8}", flush=True)
    inp, d, ref, _ = check_workload(wl, quantize_queries=q8)
    if not q8:
        idx = dsa.indexer_topk(paged_cache(d), d["q_idx"], d["w"], wl.top_k,
                               max_seq_len=int(inp.seq_lens.max()),
                               q_pos=d["q_pos"])
        torch.cuda.synchronize()
        rows = [(b, t) for b in range(wl.B) for t in range(wl.T)]
        assert_idx_equal(idx.cpu().numpy(), ref["idx"], rows)
