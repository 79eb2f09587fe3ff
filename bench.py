"""Benchmark of the DSA decode step on one MI355X.

One step = indexer -> Top-K -> sparse attention for a batch of 32 decode
tokens, each over a 32768-token bf16 cache, top_k = 2048, 64 indexer heads of
width 128 and 128 MLA heads of width 576 (512 + 64), through
dsa_decode_step on the caller's stream.  Inputs are seeded synthetic tensors
resident in HBM before the timed region; three input replicas rotate so that
consecutive steps never find their operands in the 256 MB Infinity Cache.

Prints ONE JSON line: throughput in tokens/s, the step's algorithmic HBM
bandwidth against the 8 TB/s peak, the roofline of the dominant kernel (the
indexer stream, timed with HIP events on its own stream), and the CPU oracle
timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0   # dense bf16 matrix-core peak of one MI355X
PEAK_FP8_TFLOPS = 5000.0    # dense fp8 matrix-core peak of one MI355X
METRIC = ("DSA decode tokens/sec at B=32,L=32K,k=2048; achieved HBM GB/s vs "
          "peak")
REPLICAS = 3


def algorithmic_bytes(wl, L):
    """Bytes the method must move per decode step (whole batch): every
    indexer key once, every selected latent row once, the queries, weights,
    indices and outputs.  The score round-trip between kernels is excluded."""
    per_tok = (L * wl.d_I * 2                      # indexer keys, bf16
               + wl.top_k * 576 * 2                # selected latent rows
               + wl.H_I * wl.d_I * 2 + wl.H_I * 4  # q_I, w
               + wl.H * 576 * 2                    # q
               + wl.H * 512 * 4 + wl.H * 4         # out, lse
               + wl.top_k * 4)                     # indices
    return wl.B * wl.T * per_tok


def step_bytes_general(wl, lens):
    """Algorithmic bytes of one decode step over sequences of lengths `lens`
    (one query each): every indexer key (bf16, or e4m3 codes + e8m0 block
    scales) once, every selected latent row (bf16, or MXFP8 codes + scales)
    once, plus queries, weights, indices and outputs."""
    key_b = wl.d_I + wl.d_I // 32 if wl.quantized else 2 * wl.d_I
    row_b = 576 + 18 if wl.quantized else 2 * 576
    tot = 0
    for L in lens:
        L = int(L)
        tot += (L * key_b + min(wl.top_k, L) * row_b
                + wl.H_I * wl.d_I * 2 + wl.H_I * 4 + wl.H * 576 * 2
                + wl.H * 512 * 4 + wl.H * 4 + wl.top_k * 4)
    return tot


def decode_config(name, stream, steps=20, warmup=5, oracle_budget_s=0.0,
                  quantize_queries=False):
    """ms per dsa_decode_step call for another decode configuration, with
    enough input replicas rotating that a step's operands (over 1 GB in
    total) are not served from the 256 MB Infinity Cache.  quantize_queries:
    the fully quantised indexer (MX keys only)."""
    import torch
    import indexed_sparse_attention_lightning_amd as dsa
    import workloads as wk
    from workloads.device import to_device
    wl = wk.WORKLOADS[name]
    inp = wk.generate(wl)
    lens = [int(x) for x in inp.seq_lens]
    sb = step_bytes_general(wl, lens)
    nrep = max(3, -(-(1 << 30) // sb))
    base = to_device(inp)
    reps = [base] + [{k: (None if v is None else v.clone())
                      for k, v in base.items() if not k.endswith("_c")}
                     for _ in range(nrep - 1)]
    caches = [dsa.PagedCache(kidx=d["kidx"], kv=d["kv"],
                             page_table=d["page_table"], seq_lens=d["seq_lens"],
                             kidx_scale=d["kidx_scale"], kv_scale=d["kv_scale"])
              for d in reps]
    max_len = max(lens)
    ws = torch.empty(dsa.workspace_size(dsa.OP_DECODE_STEP, wl.B, 1, max_len,
                                        wl.H, wl.top_k), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty((wl.B, 1, wl.H, 512), device="cuda")
    l = torch.empty((wl.B, 1, wl.H), device="cuda")

    def step(i):
        r = i % nrep
        d = reps[r]
        dsa.decode_step(caches[r], d["q_idx"], d["w"], d["q"], wl.top_k,
                        wl.softmax_scale, max_seq_len=max_len, out=o, lse=l,
                        workspace=ws, quantize_queries=quantize_queries)

    ms = time_loop(step, steps, warmup, stream)
    gbps = sb / (ms * 1e-3) / 1e9
    res = {"ms_per_step": round(ms, 5),
           "tokens_per_s": round(wl.B / (ms * 1e-3), 1),
           "step_algorithmic_bytes": sb,
           "step_hbm_gbps": round(gbps, 1),
           "step_frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4),
           "input_replicas": nrep}
    del reps, caches, base, ws
    torch.cuda.empty_cache()
    if oracle_budget_s > 0:
        res["cpu_oracle"] = oracle_rate(inp, oracle_budget_s,
                                        quantize_queries=quantize_queries)
    return res


def t128_step_bytes(wl, lens):
    """Algorithmic bytes of one decode step over a cache of MX block-32
    indexer keys and 128-tile latent KV (576 codes + 5 fp32 scales a row)."""
    tot = 0
    for L in lens:
        L = int(L)
        tot += (L * (wl.d_I + wl.d_I // 32) + min(wl.top_k, L) * (576 + 20)
                + wl.H_I * wl.d_I * 2 + wl.H_I * 4 + wl.H * 576 * 2
                + wl.H * 512 * 4 + wl.H * 4 + wl.top_k * 4)
    return tot


def decode_t128_config(stream, steps=20, warmup=5, oracle_budget_s=0.0):
    """The decode batch (32 x 32768, top_k 2048) over a cache written by
    dsa_cache_append from the bf16 rows: MX block-32 indexer keys and the
    128-tile latent KV.  Times the decode step (rotating input replicas past
    the Infinity Cache), the append of one new token per sequence, and the
    append of the whole cache (1M tokens, the kernel's streaming rate)."""
    import dataclasses
    import torch
    import indexed_sparse_attention_lightning_amd as dsa
    import oracle
    import workloads as wk
    from workloads.device import to_device
    wl = wk.WORKLOADS["decode"]
    inp = wk.generate(wl)
    B, L = wl.B, inp.L
    sb = t128_step_bytes(wl, [L] * B)
    nrep = max(3, -(-(1 << 30) // sb))
    base = to_device(inp)
    P = base["kv"].shape[0]
    pos = torch.arange(L, dtype=torch.int32, device="cuda").repeat(B, 1)
    k_rows = base["kidx"].view(B, L, wl.d_I)
    v_rows = base["kv"].view(B, L, 576)

    def new_cache():
        return dsa.PagedCache(
            kidx=torch.empty((P, 64, wl.d_I), dtype=torch.uint8, device="cuda"),
            kv=torch.empty((P, 64, 576), dtype=torch.uint8, device="cuda"),
            page_table=base["page_table"], seq_lens=base["seq_lens"],
            kidx_scale=torch.empty((P, 64, wl.d_I // 32), dtype=torch.uint8,
                                   device="cuda"),
            kv_scale=torch.empty((P, 64, 5), dtype=torch.float32,
                                 device="cuda"))

    caches = []
    for _ in range(nrep):
        c = new_cache()
        dsa.cache_append(c, pos, k_new=k_rows, kv_new=v_rows)
        caches.append(c)
    torch.cuda.synchronize()
    ws = torch.empty(dsa.workspace_size(dsa.OP_DECODE_STEP, B, 1, L, wl.H,
                                        wl.top_k), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty((B, 1, wl.H, 512), device="cuda")
    lse = torch.empty((B, 1, wl.H), device="cuda")
    ms = time_loop(lambda i: dsa.decode_step(
        caches[i % nrep], base["q_idx"], base["w"], base["q"], wl.top_k,
        wl.softmax_scale, max_seq_len=L, out=o, lse=lse, workspace=ws),
        steps, warmup, stream)
    # one new token per sequence (the last position, rewritten in place)
    last = pos[:, -1:].contiguous()
    k1 = k_rows[:, -1:].contiguous()
    v1 = v_rows[:, -1:].contiguous()
    ms_app1 = time_loop(lambda i: dsa.cache_append(
        caches[i % nrep], last, k_new=k1, kv_new=v1), steps, warmup, stream)
    ms_bulk = time_loop(lambda i: dsa.cache_append(
        caches[i % nrep], pos, k_new=k_rows, kv_new=v_rows), 5, 2, stream)
    bulk_bytes = B * L * (wl.d_I * 2 + 576 * 2 + 4          # read: rows, pos
                          + wl.d_I + wl.d_I // 32 + 576 + 20)  # written
    bulk_gbps = bulk_bytes / (ms_bulk * 1e-3) / 1e9
    gbps = sb / (ms * 1e-3) / 1e9
    res = {"ms_per_step": round(ms, 5),
           "tokens_per_s": round(B / (ms * 1e-3), 1),
           "step_algorithmic_bytes": sb,
           "step_hbm_gbps": round(gbps, 1),
           "step_frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4),
           "input_replicas": nrep,
           "cache_append": {
               "one_token_per_sequence_us": round(ms_app1 * 1e3, 2),
               "whole_cache_ms": round(ms_bulk, 4),
               "whole_cache_tokens": B * L,
               "whole_cache_algorithmic_bytes": bulk_bytes,
               "whole_cache_hbm_gbps": round(bulk_gbps, 1),
               "whole_cache_frac_of_peak": round(bulk_gbps / PEAK_HBM_GBPS, 4)}}
    del caches, ws, base, k_rows, v_rows
    torch.cuda.empty_cache()
    if oracle_budget_s > 0:
        # the oracle's own quantisation of the first two sequences' rows
        sub = 2
        npg = sub * L // 64
        kd, ks = oracle.quantize_rows(inp.k_idx.data[:npg], "mx32")
        vd, vs = oracle.quantize_rows(inp.kv.data[:npg], "t128")
        wl_s = dataclasses.replace(wl, B=sub)
        inp_s = dataclasses.replace(
            inp, wl=wl_s, seq_lens=inp.seq_lens[:sub], q_pos=inp.q_pos[:sub],
            page_table=inp.page_table[:sub], q_idx=inp.q_idx[:sub],
            w=inp.w[:sub], q=inp.q[:sub], k_idx=wk.Cache(kd, ks, True),
            kv=wk.Cache(vd, vs, "t128"))
        res["cpu_oracle"] = oracle_rate(inp_s, oracle_budget_s)
    return res


def indexer_bytes(wl, L):
    """Algorithmic bytes of one indexer launch: keys + queries + weights."""
    return wl.B * wl.T * (L * wl.d_I * 2 + wl.H_I * wl.d_I * 2 + wl.H_I * 4)


def time_loop(fn, steps, warmup, stream, per_call=False):
    """Mean ms per call over `steps` back-to-back calls on `stream` (events
    around the whole loop); with per_call also the 10th/50th/90th percentile
    of the calls, each bracketed by its own event pair."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        fn(i)
    end.record(stream)
    torch.cuda.synchronize()
    mean = start.elapsed_time(end) / steps
    if not per_call:
        return mean
    ev = [(torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        fn(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev])
    return mean, {"p10": round(float(np.percentile(t, 10)), 5),
                  "p50": round(float(np.percentile(t, 50)), 5),
                  "p90": round(float(np.percentile(t, 90)), 5)}


def traffic_record(kernel_src):
    """HBM bytes per indexer launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "indexer_stream_decode_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()
    if rec.get("kernel_source_sha256") != h:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(inp, budget_s=12.0):
    """The CPU oracle, as it stands, on whole decode rows of the same
    workload (every row of the batch, in passes over it) until about
    `budget_s` seconds of work."""
    import contextlib
    import oracle
    # the host's cores as this process may use them; BLAS threads set to it
    cores = len(os.sched_getaffinity(0))
    blas = None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        ctx = threadpool_limits(limits=cores, user_api="blas")
    except Exception:  # pragma: no cover
        ctx = contextlib.nullcontext()
    with ctx:
        try:
            blas = max(i.get("num_threads", 0) for i in threadpool_info()
                       if i.get("user_api") == "blas")
        except Exception:  # pragma: no cover
            blas = None
        rows, t0 = 0, time.perf_counter()
        while True:
            for b in range(inp.wl.B):
                oracle.decode_path(inp, rows=[(b, 0)])
                rows += 1
                if time.perf_counter() - t0 > budget_s:
                    break
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
    return {"value": rows / dt, "unit": "tokens/s", "cores": cores,
            "blas_threads": blas, "kind": "oracle",
            "sample": f"{rows} decode tokens ({rows / inp.wl.B:.1f} passes "
                      f"over the batch of {inp.wl.B}; full indexer over "
                      f"{inp.L} keys, top-k, attention), {dt:.1f} s"}


def oracle_rate(inp, budget_s=4.0, quantize_queries=False):
    """The CPU oracle on whole query rows of `inp` (rows in order, cycling)
    for about `budget_s` seconds: query rows per second."""
    import oracle
    allrows = [(b, t) for b in range(inp.wl.B) for t in range(inp.wl.T)]
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        oracle.decode_path(inp, rows=[allrows[n % len(allrows)]],
                           quantize_queries=quantize_queries)
        n += 1
    dt = time.perf_counter() - t0
    return {"value": round(n / dt, 2), "unit": "query rows/s",
            "kind": "oracle", "sample": f"{n} query rows, {dt:.1f} s"}


def prefill_kernels(stream, steps=5, warmup=2, oracle_budget_s=0.0,
                    quantized=False, from_start=False):
    """The prefill chunk (4096 queries at positions 61440..65535 of a
    65536-token bf16 context, 64 indexer heads x 128, top_k 2048, 128 MLA
    heads) through the three separate entry points, each timed on its own.
    The indexer is the dense contraction here: its rate is reported against
    the matrix-core peak of its operand type, with the causal (query, key)
    pairs as work.  quantized: MX keys and KV, and the fully quantised
    indexer (queries to MX block-32, scaled FP8 products, FP8 peak)."""
    import dataclasses
    import torch
    import indexed_sparse_attention_lightning_amd as dsa
    import workloads as wk
    from workloads.device import to_device

    wl = wk.WORKLOADS["prefill"]
    if quantized:
        wl = dataclasses.replace(wl, quantized=True)
    if from_start:
        wl = dataclasses.replace(wl, L=4096, first_pos=0)
    inp = wk.generate(wl)
    d = to_device(inp)
    L = inp.L
    scores = torch.empty((1, wl.T, L), device="cuda")
    idx = torch.empty((1, wl.T, wl.top_k), dtype=torch.int32, device="cuda")
    out = torch.empty((1, wl.T, wl.H, 512), device="cuda")
    lse = torch.empty((1, wl.T, wl.H), device="cuda")
    ws = torch.empty(max(1, dsa.workspace_size(dsa.OP_SPARSE_MLA, 1, wl.T, L,
                                               wl.H, wl.top_k)),
                     dtype=torch.uint8, device="cuda")
    ms_i = time_loop(lambda i: dsa.indexer_scores(
        d["q_idx"], d["w"], d["kidx_c"], d["q_pos"], out=scores,
        k_scale=d["kidx_scale_c"], quantize_queries=quantized),
        steps, warmup, stream)
    ms_t = time_loop(lambda i: dsa.topk(scores, d["q_pos"], wl.top_k,
                                        out=idx), steps, warmup, stream)
    ms_a = time_loop(lambda i: dsa.sparse_mla_attn(
        d["q"], d["kv_c"], idx, wl.softmax_scale, out=out, lse=lse,
        kv_scale=d["kv_scale_c"], workspace=ws), steps, warmup, stream)
    pairs = int(np.sum(inp.q_pos.astype(np.int64) + 1))
    idx_flop = pairs * 2 * wl.H_I * wl.d_I
    # attention work over the selected rows only (a causal row shorter than
    # top_k selects all of its positions)
    sel = int(np.sum(np.minimum(inp.q_pos.astype(np.int64) + 1, wl.top_k)))
    attn_flop = sel * wl.H * 2 * (576 + 512)
    idx_tf = idx_flop / (ms_i * 1e-3) / 1e12
    attn_tf = attn_flop / (ms_a * 1e-3) / 1e12
    ipeak = PEAK_FP8_TFLOPS if quantized else PEAK_BF16_TFLOPS
    where = ("0..4095 of a 4096" if from_start else
             "61440..65535 of a 65536")
    return {
        "workload": (f"prefill chunk: 4096 queries at {where} context, "
                     "top_k 2048, " +
                     ("MX keys and KV, quantised indexer queries (scaled FP8 "
                      "products)" if quantized else "bf16")),
        "indexer_ms": round(ms_i, 4), "topk_ms": round(ms_t, 4),
        "sparse_mla_attn_ms": round(ms_a, 4),
        "indexer_roofline": {"bound": "mfma", "achieved": round(idx_tf, 1),
                             "peak": ipeak, "unit": "TFLOP/s",
                             "frac": round(idx_tf / ipeak, 4),
                             "algorithmic_flop": idx_flop},
        "attn_tflops": round(attn_tf, 1),
        "attn_frac_of_bf16_peak": round(attn_tf / PEAK_BF16_TFLOPS, 4),
        **({"cpu_oracle": oracle_rate(inp, oracle_budget_s,
                                      quantize_queries=quantized)}
           if oracle_budget_s > 0 else {}),
        "tokens_per_s": round(wl.T / ((ms_i + ms_t + ms_a) * 1e-3), 1),
    }


def fused_comparison(stream, steps=20, warmup=5):
    """dsa_indexer_topk (scoring and Top-K in one kernel, the scores kept in
    LDS) against dsa_indexer_scores followed by dsa_topk (scores through
    HBM), on the bf16 decode batch's shape (32 rows of 32768) and on 256 rows
    of 4096 (the same key bytes, one row per CU), bf16 keys and MX block-32
    e4m3 keys, the latter also with the fully quantised indexer.
    Integer-valued keys and queries in [-4, 4] (exact in e4m3 with unit
    scales), power-of-two weights; both paths' indices compared."""
    import torch
    import indexed_sparse_attention_lightning_amd as dsa
    res = {}
    for B, L, mx, q8 in ((32, 32768, False, False), (256, 4096, False, False),
                         (256, 4096, True, False), (256, 4096, True, True)):
        P, K, d_I, H_I = B * L // 64, 2048, 128, 64
        g = torch.Generator(device="cuda")
        g.manual_seed(B)
        vals = torch.randint(-4, 5, (P, 64, d_I), device="cuda", generator=g)
        kscale = kc_scale = None
        if mx:
            kidx = vals.float().to(torch.float8_e4m3fn).view(torch.uint8)
            kscale = torch.full((P, 64, d_I // 32), 127, dtype=torch.uint8,
                                device="cuda")
            kc_scale = kscale.view(B, L, d_I // 32)
        else:
            kidx = vals.to(torch.bfloat16)
        del vals
        kv = torch.empty((P, 64, 576), dtype=torch.bfloat16, device="cuda")
        pt = torch.arange(P, dtype=torch.int32, device="cuda").view(B, -1)
        sl = torch.full((B,), L, dtype=torch.int32, device="cuda")
        q_idx = torch.randint(-4, 5, (B, 1, H_I, d_I), device="cuda",
                              generator=g).to(torch.bfloat16)
        w = torch.pow(2.0, -torch.randint(0, 4, (B, 1, H_I), device="cuda",
                                          generator=g).float())
        q_pos = (sl - 1).view(B, 1).contiguous()
        cache = dsa.PagedCache(kidx=kidx, kv=kv, page_table=pt, seq_lens=sl,
                               kidx_scale=kscale)
        i1 = torch.empty((B, 1, K), dtype=torch.int32, device="cuda")
        i2 = torch.empty_like(i1)
        scores = torch.empty((B, 1, L), dtype=torch.float32, device="cuda")
        kc = kidx.view(B, L, d_I)

        def fused(i):
            dsa.indexer_topk(cache, q_idx, w, K, L, q_pos=q_pos, idx_out=i1,
                             quantize_queries=q8)

        def two(i):
            dsa.indexer_scores(q_idx, w, kc, q_pos, k_scale=kc_scale,
                               out=scores, quantize_queries=q8)
            dsa.topk(scores, q_pos, K, out=i2)

        ms_f = time_loop(fused, steps, warmup, stream)
        ms_2 = time_loop(two, steps, warmup, stream)
        torch.cuda.synchronize()
        kbytes = B * L * (d_I + d_I // 32 if mx else d_I * 2)
        res[f"{B}x{L}" + ("_mx" if mx else "") + ("_q8" if q8 else "")] = {
            "fused_us": round(ms_f * 1e3, 2),
            "indexer_then_topk_us": round(ms_2 * 1e3, 2),
            "fused_key_gbps": round(kbytes / (ms_f * 1e-3) / 1e9, 1),
            "same_idx": bool(torch.equal(i1, i2))}
        del kidx, kv, scores, cache, kscale, kc_scale
        torch.cuda.empty_cache()
    return res


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill-chunk kernel timings")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the FP8 and ragged decode configurations")
    ap.add_argument("--only-config",
                    choices=["decode_fp8", "decode_fp8_q8", "ragged", "fused",
                             "decode_t128", "prefill", "prefill_quantized",
                             "prefill_from_start"],
                    help="time only this decode configuration (10 steps after "
                         "3 warm-up steps) and print its JSON object; for "
                         "kernel traces")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip the fused indexer + Top-K comparison")
    ap.add_argument("--kernels-only", action="store_true",
                    help="run one 256 MiB device copy (counter calibration) "
                         "and one decode step, then exit (for rocprofv3 "
                         "--pmc runs)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU only: the DSA hot path here is a "
              "single-GPU kernel set (decode batches shard by sequence with "
              "no exchange); run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    import indexed_sparse_attention_lightning_amd as dsa
    import workloads as wk
    from workloads.device import to_device

    if args.only_config:
        st = torch.cuda.current_stream()
        if args.only_config == "fused":
            res = fused_comparison(st)
        elif args.only_config.startswith("prefill"):
            res = prefill_kernels(
                st, quantized=args.only_config == "prefill_quantized",
                from_start=args.only_config == "prefill_from_start")
        elif args.only_config == "decode_t128":
            res = decode_t128_config(st, steps=10, warmup=3)
        elif args.only_config == "decode_fp8_q8":
            res = decode_config("decode_fp8", st, steps=10, warmup=3,
                                quantize_queries=True)
        else:
            res = decode_config(args.only_config, st, steps=10, warmup=3)
        print(json.dumps({"config": args.only_config, **res}), flush=True)
        return 0

    wl = wk.WORKLOADS["decode"]
    inp = wk.generate(wl)
    L = inp.L
    reps = [to_device(inp)]
    for _ in range(REPLICAS - 1):
        d = {k: (None if v is None else v.clone())
             for k, v in reps[0].items() if not k.endswith("_c")}
        d["kidx_c"] = d["kidx"].view(wl.B, L, wl.d_I)
        d["kv_c"] = d["kv"].view(wl.B, L, 576)
        reps.append(d)
    stream = torch.cuda.current_stream()
    caches = [dsa.PagedCache(kidx=d["kidx"], kv=d["kv"],
                             page_table=d["page_table"],
                             seq_lens=d["seq_lens"]) for d in reps]
    ws = torch.empty(dsa.workspace_size(dsa.OP_DECODE_STEP, wl.B, 1, L, wl.H,
                                        wl.top_k), dtype=torch.uint8,
                     device="cuda")
    outs = [(torch.empty((wl.B, 1, wl.H, 512), device="cuda"),
             torch.empty((wl.B, 1, wl.H), device="cuda"),
             torch.empty((wl.B, 1, wl.top_k), dtype=torch.int32,
                         device="cuda")) for _ in range(REPLICAS)]

    def step(i):
        r = i % REPLICAS
        d = reps[r]
        o, l, ix = outs[r]
        dsa.decode_step(caches[r], d["q_idx"], d["w"], d["q"], wl.top_k,
                        wl.softmax_scale, max_seq_len=L, out=o, lse=l,
                        idx_out=ix, workspace=ws)

    if args.kernels_only:
        torch.cuda.synchronize()
        src = torch.ones(1 << 26, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)                  # reads and writes exactly 256 MiB
        torch.cuda.synchronize()
        step(0)
        torch.cuda.synchronize()
        print(json.dumps({"kernels_only": True, "copy_bytes": 1 << 28}))
        return 0

    ms, ms_pct = time_loop(step, args.steps, args.warmup, stream,
                           per_call=True)

    # the same steps replayed from HIP graphs (one captured step per replica)
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for r in range(REPLICAS):
            step(r)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    for r in range(REPLICAS):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(r)
        graphs.append(g)
    torch.cuda.synchronize()
    ms_graph = time_loop(lambda i: graphs[i % REPLICAS].replay(), args.steps,
                         args.warmup, stream)
    del graphs

    # per-kernel timing of the three stages through the separate entry points
    scores = [torch.empty((wl.B, 1, L), device="cuda") for _ in range(REPLICAS)]

    def ix_call(i):
        r = i % REPLICAS
        dsa.indexer_scores(reps[r]["q_idx"], reps[r]["w"], reps[r]["kidx_c"],
                           reps[r]["q_pos"], out=scores[r])

    ms_idx = time_loop(ix_call, args.steps, args.warmup, stream)

    def tk_call(i):
        r = i % REPLICAS
        dsa.topk(scores[r], reps[r]["q_pos"], wl.top_k, out=outs[r][2])

    ms_topk = time_loop(tk_call, args.steps, args.warmup, stream)
    attn_ws = torch.empty(max(1, dsa.workspace_size(
        dsa.OP_SPARSE_MLA, wl.B, 1, L, wl.H, wl.top_k)), dtype=torch.uint8,
        device="cuda")

    def at_call(i):
        r = i % REPLICAS
        dsa.sparse_mla_attn(reps[r]["q"], reps[r]["kv_c"], outs[r][2],
                            wl.softmax_scale, out=outs[r][0], lse=outs[r][1],
                            workspace=attn_ws)

    ms_attn = time_loop(at_call, args.steps, args.warmup, stream)

    # a plain device copy of a 1 GiB buffer: the practical streaming ceiling
    a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    bcopy = torch.empty_like(a)
    ms_copy = time_loop(lambda i: bcopy.copy_(a), 10, 3, stream)
    copy_gbps = 2 * a.numel() * 4 / (ms_copy * 1e-3) / 1e9
    del a, bcopy

    step_bytes = algorithmic_bytes(wl, L)
    tok_s = wl.B * wl.T / (ms * 1e-3)
    step_gbps = step_bytes / (ms * 1e-3) / 1e9
    ib = indexer_bytes(wl, L)
    idx_gbps = ib / (ms_idx * 1e-3) / 1e9
    src = os.path.join(ROOT, "indexed_sparse_attention_lightning_amd", "csrc",
                       "indexer.hip")
    line = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "ms_per_step_percentiles": ms_pct,
        "ms_per_step_graph_replay": round(ms_graph, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "decode_bf16: batch 32, every sequence at 32768 "
                        "cached tokens, top_k 2048, indexer 64 heads x 128, "
                        "MLA 128 heads x (512+64), bf16 cache read through "
                        "an identity page table",
            "global_batch": wl.B, "seq_len": L, "top_k": wl.top_k,
            "parallelism": "single GPU"},
        "step_hbm_gbps": round(step_gbps, 1),
        "step_frac_of_peak": round(step_gbps / PEAK_HBM_GBPS, 4),
        "step_algorithmic_bytes": step_bytes,
        "kernel_ms": {"indexer": round(ms_idx, 5), "topk": round(ms_topk, 5),
                      "sparse_mla_attn": round(ms_attn, 5)},
        "copy_gbps_measured": round(copy_gbps, 1),
        "roofline": {
            "kernel": "indexer_stream_kernel (dsa_indexer_scores)",
            "bound": "hbm", "achieved": round(idx_gbps, 1),
            "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(idx_gbps / PEAK_HBM_GBPS, 4),
            "traffic": traffic_record(src),
            "algorithmic_bytes_per_launch": ib},
    }
    del reps, caches, outs, scores
    if not args.no_fused:
        line["fused_indexer_topk"] = fused_comparison(stream)
    if not args.no_prefill:
        line["prefill"] = prefill_kernels(
            stream, oracle_budget_s=0 if args.no_cpu_baseline else 4.0)
        line["prefill_quantized"] = prefill_kernels(
            stream, oracle_budget_s=0 if args.no_cpu_baseline else 4.0,
            quantized=True)
        line["prefill_from_start"] = prefill_kernels(
            stream, oracle_budget_s=0 if args.no_cpu_baseline else 4.0,
            from_start=True)
    if not args.no_configs:
        line["other_configs"] = {
            "decode_fp8": dict(workload="batch 32 x 32768, e4m3 indexer keys "
                               "and MXFP8 latent KV (block 32, e8m0 scales), "
                               "top_k 2048", **decode_config(
                                   "decode_fp8", stream,
                                   oracle_budget_s=0 if args.no_cpu_baseline else 4.0)),
            "decode_fp8_q8": dict(workload="the FP8 decode batch with the "
                                  "fully quantised indexer: queries to MX "
                                  "block-32 on the fly, scaled FP8 matrix "
                                  "cores over the e4m3 keys", **decode_config(
                                      "decode_fp8", stream, oracle_budget_s=0
                                      if args.no_cpu_baseline else 4.0,
                                      quantize_queries=True)),
            "ragged": dict(workload="batch 4, lengths uniform in [16384, "
                           "131072], 64-token pages scattered by a seeded "
                           "page table, FP8 keys and MXFP8 KV, top_k 2048",
                           **decode_config(
                               "ragged", stream,
                               oracle_budget_s=0 if args.no_cpu_baseline else 4.0)),
            "decode_t128": dict(workload="batch 32 x 32768, top_k 2048, cache "
                                "written by dsa_cache_append: MX block-32 "
                                "indexer keys, latent KV as e4m3 with one fp32 "
                                "scale per 128-feature tile",
                                **decode_t128_config(
                                    stream, oracle_budget_s=0
                                    if args.no_cpu_baseline else 4.0)),
        }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
