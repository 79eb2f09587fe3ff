"""HIP path vs CPU oracle, through the C ABI (needs an MI355X).

Top-K index sets must match exactly; indexer scores bit-exactly (integer
inputs make them exact in fp32); attention outputs within
max|diff| <= 1e-2 * max|oracle| and LSE within 1e-3.
"""
import numpy as np
import pytest
import torch

import indexed_sparse_attention_lightning_amd as dsa
import oracle
import workloads as wk
from workloads.device import to_device

from gpu_helpers import (assert_attn_close, assert_idx_equal, check_workload,
                         prefill_rows, run_decode_step, run_separate_ops)

pytestmark = pytest.mark.gpu

W = wk.WORKLOADS


def test_tiny_workload():
    """Batch 1, position 511 over L=512, H_I=4, d_I=64, K=64, 16 heads."""
    check_workload(W["tiny"])


# Reduced shapes: several tiles, ragged tails, both cache formats, paging.
SMALL = {
    "decode_bf16": wk.scaled(W["decode"], B=3, L=2048, top_k=256, seed=101),
    "decode_fp8": wk.scaled(W["decode_fp8"], B=3, L=2048, top_k=256, seed=101),
    "decode_ragged_tail": wk.scaled(W["decode"], B=2, L=1000, top_k=300,
                                    seed=102),
    "prefill_chunk": wk.scaled(W["prefill"], T=40, L=1536, first_pos=1400,
                               top_k=512, H=64, seed=103),
    "paged_fp8": wk.scaled(W["ragged"], B=3, L_min=100, L_max=3000,
                           top_k=512, seed=104),
    "paged_small_heads": wk.scaled(W["ragged"], B=2, L_min=700, L_max=1300,
                                   top_k=128, H=40, H_I=20, d_I=64, seed=105),
    "odd_heads_bf16": wk.scaled(W["decode"], B=2, L=1024, top_k=96, H=100,
                                H_I=48, seed=106),
    # query-tiled indexer: a ragged last query tile, unaligned L, FP8 keys
    "prefill_ragged_fp8": wk.scaled(W["prefill"], T=37, L=1000, first_pos=900,
                                    top_k=300, H=32, quantized=True, seed=107),
    "prefill_small_dims": wk.scaled(W["prefill"], T=19, L=700, first_pos=600,
                                    top_k=128, H=16, H_I=20, d_I=64,
                                    quantized=True, seed=108),
    # few tokens, long selections: the most attention splits per token
    "few_tokens_long_k": wk.scaled(W["decode"], B=2, L=4096, top_k=2048,
                                   H=64, seed=110),
    "paged_fp8_long_k": wk.scaled(W["ragged"], B=1, L_min=3000, L_max=5000,
                                  top_k=1536, seed=111),
    # causal skipping of whole stages, rows shorter than K
    "prefill_from_start": wk.scaled(W["prefill"], T=130, L=640, first_pos=0,
                                    top_k=64, H=16, seed=109),
    # query-tiled indexer over scattered pages (its per-stage page lookups)
    "prefill_paged_scattered": wk.scaled(W["prefill"], T=24, L=1500,
                                         first_pos=1300, top_k=256, H=32,
                                         paged_random=True, seed=112),
    "prefill_paged_scattered_fp8": wk.scaled(W["prefill"], T=21, L=1300,
                                             first_pos=1100, top_k=200, H=16,
                                             quantized=True,
                                             paged_random=True, seed=113),
    # 256 tokens or more: one attention split per token (no combine, the
    # software-pipelined tile loop); a ragged last tile, heads that leave
    # one wave partly and two wholly idle, and causal rows of 1 to 3 tiles
    "prefill_nosplit": wk.scaled(W["prefill"], T=260, L=1200, first_pos=940,
                                 top_k=300, H=48, seed=114),
    "prefill_nosplit_short_rows": wk.scaled(W["prefill"], T=256, L=256,
                                            first_pos=0, top_k=96, seed=115),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_workloads(name):
    check_workload(SMALL[name])


def test_topk_covers_whole_history_is_dense_attention():
    """K larger than the history: every position is selected and the
    attention equals dense attention (the oracle's dense-equivalence pin)."""
    wl = wk.scaled(W["tiny"], top_k=1024, seed=7)
    inp, d, ref, (idx, out, lse) = check_workload(wl)
    assert idx[0, 0, :512].tolist() == list(range(512))
    assert np.all(idx[0, 0, 512:] == -1)


def test_all_zero_queries_tie_break():
    """q_I = 0 makes every score 0: ties resolve to the lowest positions."""
    wl = wk.scaled(W["decode"], B=2, L=2048, top_k=256, H=32, seed=8)
    inp = wk.generate(wl)
    inp.q_idx[:] = 0
    d = to_device(inp)
    idx, out, lse = run_decode_step(inp, d)
    for b in range(2):
        assert idx[b, 0].tolist() == list(range(256))
    ref = oracle.decode_path(inp)
    assert_attn_close(out, lse, ref, [(0, 0), (1, 0)])


def test_short_histories_and_padding():
    """Queries near the start of the cache: fewer candidates than K."""
    wl = wk.scaled(W["prefill"], T=6, L=512, first_pos=0, top_k=64, H=32,
                   seed=9)
    inp = wk.generate(wl)
    inp.q_pos[0] = [0, 1, 2, 31, 63, 64]
    d = to_device(inp)
    ref = oracle.decode_path(inp, want_scores=True)
    rows = [(0, t) for t in range(6)]
    idx, out, lse = run_decode_step(inp, d)
    assert_idx_equal(idx, ref["idx"], rows)
    assert_attn_close(out, lse, ref, rows)
    scores, idx2, out2, lse2 = run_separate_ops(inp, d)
    assert_idx_equal(idx2, ref["idx"], rows)
    assert_attn_close(out2, lse2, ref, rows)
    assert np.all(idx[0, 0, 1:] == -1) and idx[0, 0, 0] == 0


def test_invalid_indices_are_skipped():
    """-1 entries in idx contribute nothing to the attention."""
    wl = wk.scaled(W["decode"], B=2, L=1024, top_k=128, H=32, seed=10)
    inp = wk.generate(wl)
    d = to_device(inp)
    rng = np.random.default_rng(0)
    idx = np.full((2, 1, 128), -1, dtype=np.int32)
    for b in range(2):
        sel = np.sort(rng.choice(1024, size=50, replace=False))
        idx[b, 0, rng.choice(128, size=50, replace=False)] = sel
    out, lse = dsa.sparse_mla_attn(d["q"], d["kv_c"],
                                   torch.from_numpy(idx).cuda(),
                                   wl.softmax_scale)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for b in range(2):
        chosen = idx[b, 0][idx[b, 0] >= 0]
        kv = oracle.cache_rows(inp.kv.data, None, False, inp.page_table[b],
                               chosen)
        ro, rl = oracle.sparse_mla_row(oracle.decode_bf16(inp.q[b, 0]), kv,
                                       wl.softmax_scale)
        assert np.abs(out[b, 0] - ro).max() <= 1e-2 * np.abs(ro).max()
        assert np.abs(lse[b, 0] - rl).max() <= 1e-3


def test_deterministic():
    wl = SMALL["paged_fp8"]
    inp = wk.generate(wl)
    d = to_device(inp)
    a = run_decode_step(inp, d)
    b = run_decode_step(inp, d)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# ------------------------------------------------------- full-size workloads

def test_full_decode_bf16():
    """B=32, L=32768, K=2048, 128 heads: every row checked."""
    check_workload(W["decode"])


def test_full_decode_fp8():
    inp, d, ref, (idx, out, lse) = check_workload(W["decode_fp8"])


def test_full_prefill_sampled_rows():
    """4096 queries at 61440..65535 of a 65536 context; 64 rows sampled:
    every position of the 8-query tile at both ends of the chunk, the rows
    around a multiple of 2048, and seeded others."""
    rows = prefill_rows()
    assert len(rows) == 64
    check_workload(W["prefill"], rows=rows, separate=True)


@pytest.mark.parametrize("quantized", [False, True])
def test_prefill_key_chunks_off_power_of_two(quantized):
    """A mid-size prefill step (2 x 1200 queries at 7760..8959 of an 8960
    context): the query-tiled indexers cut each tile's keys into chunks
    sized for about two workgroups per CU, here 5376 keys, so every causal
    row crosses a chunk boundary that is no multiple of 2048.  Sampled rows
    of both sequences through the decode step and the separate entry points:
    scores bit for bit, indices exactly, attention within tolerance; bf16
    keys, or MX keys with the quantised indexer."""
    wl = wk.scaled(W["prefill"], B=2, T=1200, L=8960, first_pos=7760,
                   top_k=256, H=16, quantized=quantized,
                   seed=131 if quantized else 130)
    rows = [(b, t) for b in range(2)
            for _, t in prefill_rows(T=1200, seed=78 + b, n_random=40)]
    assert len(rows) == 2 * 72
    check_workload(wl, rows=rows, separate=True, quantize_queries=quantized)


def test_full_ragged_paged():
    check_workload(W["ragged"])


@pytest.mark.parametrize("T,first_pos", [(1, None), (21, 950)])
def test_contiguous_api_unaligned_length(T, first_pos):
    """Separate entry points over a contiguous cache whose length is not a
    multiple of the key stage (the last stage is clamped in-bounds); T=1 runs
    the streaming indexer, T=21 the query-tiled one with a ragged tile."""
    if T == 1:
        wl = wk.scaled(W["decode"], B=2, L=1000, top_k=200, H=64, seed=11)
    else:
        wl = wk.scaled(W["prefill"], B=2, T=T, L=1000, first_pos=first_pos,
                       top_k=200, H=64, seed=12)
    inp = wk.generate(wl)
    d = to_device(inp)
    B, L = 2, 1000
    kidx_c = d["kidx"].view(B, -1, wl.d_I)[:, :L].contiguous()
    kv_c = d["kv"].view(B, -1, 576)[:, :L].contiguous()
    ref = oracle.decode_path(inp, want_scores=True)
    scores = dsa.indexer_scores(d["q_idx"], d["w"], kidx_c, d["q_pos"])
    idx = dsa.topk(scores, d["q_pos"], wl.top_k)
    out, lse = dsa.sparse_mla_attn(d["q"], kv_c, idx, wl.softmax_scale)
    torch.cuda.synchronize()
    rows = [(b, t) for b in range(B) for t in range(T)]
    sc = scores.cpu().numpy()
    for b, t in rows:
        qp = int(inp.q_pos[b, t])
        want = np.full(L, -np.inf)
        want[:qp + 1] = ref["scores"][(b, t)]
        assert np.array_equal(sc[b, t].astype(np.float64), want), (b, t)
    assert_idx_equal(idx.cpu().numpy(), ref["idx"], rows)
    assert_attn_close(out.cpu().numpy(), lse.cpu().numpy(), ref, rows)


def test_decode_rows_shorter_than_context():
    """The decode batch (32 x 32768) with some sequences far shorter than
    the context.  The indexer's waves past a row's last position leave no
    key range, and the Top-K (which takes each row's key range from the
    waves that scored it) must use only the ranges of waves with causal
    positions: rows of several lengths, one shorter than K (every position
    selected), compared with the oracle."""
    import dataclasses
    wl = W["decode"]
    inp = wk.generate(wl)
    lens = inp.seq_lens.copy()
    short = {0: 2100, 5: 9000, 17: 20000, 30: 1500, 31: 30001}
    for b, n in short.items():
        lens[b] = n
    inp = dataclasses.replace(inp, seq_lens=lens,
                              q_pos=(lens - 1).reshape(-1, 1).astype(np.int32))
    d = to_device(inp)
    rows = [(b, 0) for b in sorted(short)] + [(3, 0)]
    ref = oracle.decode_path(inp, rows=rows)
    idx, out, lse = run_decode_step(inp, d)
    assert_idx_equal(idx, ref["idx"], rows)
    assert_attn_close(out, lse, ref, rows)
    assert np.all(idx[30, 0, 1500:] == -1)


def test_indexer_long_wave_ranges():
    """Many long rows: each wave scores more than one LDS score buffer
    (several flushes per wave) and a tail shorter than a stage; queries at
    varied positions mask part of some waves' ranges.  Scores compared
    exactly with the oracle on sampled rows."""
    rng = np.random.default_rng(21)
    B, L, H_I, d_I = 40, 40001, 64, 128
    q_i = rng.integers(-4, 5, (B, 1, H_I, d_I)).astype(np.float32)
    k_i = rng.integers(-4, 5, (B, L, d_I)).astype(np.float32)
    w = np.ldexp(1.0, -rng.integers(0, 4, (B, 1, H_I))).astype(np.float32)
    q_pos = np.full((B, 1), L - 1, dtype=np.int32)
    q_pos[1, 0], q_pos[2, 0], q_pos[3, 0] = 12345, 0, 33000
    to_bf16 = lambda x: torch.from_numpy(
        wk.f32_to_bf16_bits(x).view(np.int16)).view(torch.bfloat16)
    scores = dsa.indexer_scores(to_bf16(q_i).cuda(), torch.from_numpy(w).cuda(),
                                to_bf16(k_i).cuda(),
                                torch.from_numpy(q_pos).cuda())
    torch.cuda.synchronize()
    sc = scores.cpu().numpy()
    for b in (0, 1, 2, 3, 39):
        qp = int(q_pos[b, 0])
        want = np.full(L, -np.inf)
        want[:qp + 1] = oracle.indexer_scores_row(q_i[b, 0], w[b, 0],
                                                  k_i[b, :qp + 1])
        assert np.array_equal(sc[b, 0].astype(np.float64), want), b


# ------------------------------------------- softmax over a wide logit range

def _wide_range_inputs(B, T, H, K, seed):
    """Queries and latent rows whose logits (log2 units) spread over several
    hundred units across the selected rows, rising within every run of 128
    rows (the first 32-row tile of each run lowest, so a reference taken from
    a run's first tile is far below its later maxima) and with a permuted
    offset per run (runs end far apart in their sums).  q[h] is a_h times a
    vector of ones (a_h in 1..1.875, exact in bf16), row s is b_s times ones
    plus N(0, 0.5) noise, b_s = off[run] + 3 * (s mod 128) / 127 - 2."""
    rng = np.random.default_rng(seed)
    L = K
    a = 1.0 + (np.arange(H) % 8) / 8.0
    q = np.broadcast_to(a[None, None, :, None], (B, T, H, 576)).astype(np.float32)
    runs = (L + 127) // 128
    off = rng.permutation(np.linspace(-1.5, 1.5, runs))
    s = np.arange(L)
    b = off[s // 128] + 3.0 * (s % 128) / 127.0 - 2.0
    kv = (b[None, :, None] + 0.5 * rng.standard_normal((B, L, 576))).astype(np.float32)
    idx = np.broadcast_to(np.arange(K, dtype=np.int32), (B, T, K)).copy()
    return wk.f32_to_bf16_bits(q), kv, idx


@pytest.mark.parametrize("B,T,H,K,fmt", [
    (2, 1, 128, 2048, "bf16"),     # 16 splits per token, combined by LSE
    (2, 1, 128, 2048, "mx32"),
    (1, 256, 64, 128, "bf16"),     # one split per token: no combine
])
def test_wide_logit_range(B, T, H, K, fmt):
    """Logits spread far beyond the first tile's max (well past the range a
    reference fixed at the first tile covers, so the second softmax pass
    runs) and across the splits of a token (whose partial sums then differ
    by far more than the fp32 exponent range): out and LSE against the
    oracle's fp64 softmax, element by element, and nothing NaN."""
    scale = 1.0 / np.sqrt(192.0)
    q_bits, kv_f, idx = _wide_range_inputs(B, T, H, K, seed=31 + T)
    q = torch.from_numpy(q_bits.view(np.int16)).view(torch.bfloat16).cuda()
    if fmt == "bf16":
        kv_bits = wk.f32_to_bf16_bits(kv_f)
        kv_ref = oracle.decode_bf16(kv_bits)
        kv = torch.from_numpy(kv_bits.view(np.int16)).view(torch.bfloat16).cuda()
        kv_scale = None
    else:
        codes, sc = wk.mx32_quantize(kv_f)
        kv_ref = oracle.dequant_mx32(codes, sc)
        kv = torch.from_numpy(codes).cuda()
        kv_scale = torch.from_numpy(sc).cuda()
    out, lse = dsa.sparse_mla_attn(q, kv, torch.from_numpy(idx).cuda(), scale,
                                   kv_scale=kv_scale)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    qf = oracle.decode_bf16(q_bits)
    ref_o = np.empty((B, T, H, 512))
    ref_l = np.empty((B, T, H))
    for bb in range(B):
        for t in range(T):
            ref_o[bb, t], ref_l[bb, t] = oracle.sparse_mla_row(
                qf[bb, t], kv_ref[bb, idx[bb, t]], scale)
    z = (qf[0, 0] @ kv_ref[0].T) * scale / np.log(2.0)
    assert z.max() - z.min() > 200.0   # the spread this test is about
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    err = np.abs(out - ref_o).max()
    assert err <= 1e-2 * np.abs(ref_o).max(), err
    assert np.abs(lse - ref_l).max() <= 1e-3


@pytest.mark.parametrize("case", ["few_values", "all_equal"])
def test_decode_topk_heavy_ties(case):
    """Decode rows of 32768 positions whose scores take few distinct values,
    through the decode step (the Top-K takes each row's key range from the
    indexer): with one indexer head reading one key feature, the scores are
    w * max(0, k), five values, so the K-th largest score is shared by
    thousands of positions and the lowest of them must be taken; with all
    queries zero every score is 0 and the first K positions are taken."""
    wl = wk.scaled(W["decode"], B=3, top_k=2048, H=32, seed=41)
    q = np.zeros((wl.B, wl.T, wl.H_I, wl.d_I), dtype=np.float32)
    if case == "few_values":
        q[:, :, 0, 0] = 1.0
    check_workload(wl, q_idx=wk.f32_to_bf16_bits(q), separate=False)
