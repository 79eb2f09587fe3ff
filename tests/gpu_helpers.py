"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding on seeded workloads and compare with the CPU oracle."""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import indexed_sparse_attention_lightning_amd as dsa
import oracle
import workloads as wk
from workloads.device import to_device

OUT_REL_TOL = 1e-2    # max|out - oracle| <= 1e-2 * max|oracle out|
LSE_ABS_TOL = 1e-3    # max|lse - oracle lse| <= 1e-3


def prefill_rows(T=4096, seed=77, n_random=32):
    """Sampled query rows of a prefill chunk: the first and the last eight
    (every position of the query-tiled indexer's 8-query tile, at both ends),
    the 16 around T/2 (for the 4096-query chunk at 61440..65535 these straddle
    position 63488, a multiple of 2048), and n_random seeded others: 64 rows
    for the full chunk."""
    ts = set(range(8)) | set(range(T - 8, T)) | set(range(T // 2 - 8, T // 2 + 8))
    rng = np.random.default_rng(seed)
    others = [t for t in rng.permutation(T) if t not in ts][:n_random]
    return [(0, int(t)) for t in sorted(ts | set(others))]


def paged_cache(d) -> dsa.PagedCache:
    return dsa.PagedCache(kidx=d["kidx"], kv=d["kv"], page_table=d["page_table"],
                          seq_lens=d["seq_lens"], kidx_scale=d["kidx_scale"],
                          kv_scale=d["kv_scale"])


def run_decode_step(inp, d, pass_qpos=None, quantize_queries=False):
    """The whole path through dsa_decode_step; returns numpy idx/out/lse."""
    wl = inp.wl
    use_qpos = (wl.T > 1) if pass_qpos is None else pass_qpos
    idx = torch.empty((wl.B, wl.T, wl.top_k), dtype=torch.int32, device="cuda")
    out, lse, _ = dsa.decode_step(
        paged_cache(d), d["q_idx"], d["w"], d["q"], wl.top_k, wl.softmax_scale,
        max_seq_len=int(inp.seq_lens.max()),
        q_pos=d["q_pos"] if use_qpos else None, idx_out=idx,
        quantize_queries=quantize_queries)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()


def run_separate_ops(inp, d, quantize_queries=False):
    """Indexer -> Top-K -> attention through the three separate entry points
    (contiguous caches).  Returns numpy scores/idx/out/lse."""
    wl = inp.wl
    scores = dsa.indexer_scores(d["q_idx"], d["w"], d["kidx_c"], d["q_pos"],
                                k_scale=d["kidx_scale_c"],
                                quantize_queries=quantize_queries)
    idx = dsa.topk(scores, d["q_pos"], wl.top_k)
    out, lse = dsa.sparse_mla_attn(d["q"], d["kv_c"], idx, wl.softmax_scale,
                                   kv_scale=d["kv_scale_c"])
    torch.cuda.synchronize()
    return (scores.cpu().numpy(), idx.cpu().numpy(), out.cpu().numpy(),
            lse.cpu().numpy())


def assert_idx_equal(idx, ref_idx, rows):
    for b, t in rows:
        got, want = idx[b, t], ref_idx[b, t]
        if not np.array_equal(got, want):
            bad = np.nonzero(got != want)[0]
            raise AssertionError(
                f"idx mismatch at row (b={b}, t={t}): {len(bad)} slots differ, "
                f"first at {bad[0]}: got {got[bad[0]]}, want {want[bad[0]]}")


def assert_attn_close(out, lse, ref, rows):
    o = np.stack([out[b, t] for b, t in rows]).astype(np.float64)
    ro = np.stack([ref["out"][b, t] for b, t in rows])
    l = np.stack([lse[b, t] for b, t in rows]).astype(np.float64)
    rl = np.stack([ref["lse"][b, t] for b, t in rows])
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))
    err = np.abs(o - ro).max()
    tol = OUT_REL_TOL * np.abs(ro).max()
    assert err <= tol, f"out max|diff| {err:.3e} > tol {tol:.3e}"
    lerr = np.abs(l - rl).max()
    assert lerr <= LSE_ABS_TOL, f"lse max|diff| {lerr:.3e} > {LSE_ABS_TOL}"


def check_workload(wl, rows=None, separate=None, q_idx=None,
                   quantize_queries=False):
    """Generate, run the HIP path, run the oracle on `rows`, compare.
    ``q_idx``: bf16 bits replacing the generated indexer queries;
    ``quantize_queries``: the fully quantised indexer on both sides."""
    inp = wk.generate(wl)
    if q_idx is not None:
        inp = dataclasses.replace(inp, q_idx=q_idx)
    d = to_device(inp)
    rows = rows or [(b, t) for b in range(wl.B) for t in range(wl.T)]
    ref = oracle.decode_path(inp, rows=rows, want_scores=True,
                             quantize_queries=quantize_queries)
    idx, out, lse = run_decode_step(inp, d, quantize_queries=quantize_queries)
    assert_idx_equal(idx, ref["idx"], rows)
    assert_attn_close(out, lse, ref, rows)
    if separate is None:
        separate = inp.contiguous
    if separate:
        scores, idx2, out2, lse2 = run_separate_ops(
            inp, d, quantize_queries=quantize_queries)
        L = inp.L
        for b, t in rows:
            qp = int(inp.q_pos[b, t])
            want = np.full(L, -np.inf)
            want[:qp + 1] = ref["scores"][(b, t)]
            assert np.array_equal(scores[b, t].astype(np.float64), want), \
                f"scores differ at row ({b}, {t})"
        assert_idx_equal(idx2, ref["idx"], rows)
        assert_attn_close(out2, lse2, ref, rows)
    return inp, d, ref, (idx, out, lse)
