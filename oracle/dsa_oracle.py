"""CPU oracle for the indexed sparse attention (DSA) hot path.

TEST INFRASTRUCTURE ONLY.  This module is a plain, slow, obviously correct
float64/int64 numpy statement of what the hot path computes.  Only the test
suite, the package smoke check and the benchmark's ``cpu_baseline`` leg may
import it.  The product path (the HIP library and its Python binding) never
imports, calls or falls back to it, and it shares no code with that path.

Sources (the pages are Baidu Cloud articles on Day-0 inference adaptation for
a sparse-attention architecture; "DSA" is its indexed sparse attention):

* Lightning Indexer: "relevance scoring, head-weight weighting, and Top-K
  selection" -- page "Day-0 Inference Adaptation and Performance Optimization
  for New-Architecture Large Language Models", section "Fusing the Indexer to
  Reduce Intermediate Write-Backs"; page "Day-0 Inference Optimization for a
  New Sparse Attention Architecture: A Technical Deep Dive", section 1 (LI
  scores the query against history and selects the Top-K positions) and
  section 2 ("Deep operator fusion").  The pages name the steps only; the
  score formula I[t,s] = sum_j w[t,j] * ReLU(q_I[t,j] . k_I[s]) and the
  tie-break (lower position first) are the plainest reading consistent with
  that prose and are the task's stated definition.
* Sparse Flash Attention over the selected latent KV rows, built on MLA:
  page "Inference Optimization for New Open-Source LLM Architectures",
  section "Architectural Overview" (the operator reads only the selected KV
  cache entries); same "Technical Deep Dive" page, section 1.
* Quantized caches: 8-bit float with one scale per group of 32 elements
  (page "Optimizing Inference for New Model Architectures", section 4
  "Layered Quantization"; "Technical Deep Dive" page, section 2, which names
  the format MXFP8).  Decoding follows the OCP e4m3fn / e8m0 definitions.
* Paged key cache read through a page table: "Optimizing Inference ..."
  page, section 3 ("reading the paged key cache directly").

Every function here is pinned by tests that do not re-type its formula
(brute force in pure Python, torch's fp8/bf16 decoders, torch's dense SDPA,
closed forms and invariants); none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

D_VALUE = 512          # values are the first 512 latent features


# ------------------------------------------------------------------ decoding

def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64.  bf16 is the top half of an
    IEEE binary32, so widening the bits gives the exact value."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 e4m3fn codes (uint8) -> float64, from the bit definition.

    sign(1) exponent(4, bias 7) mantissa(3); exponent field 0 encodes the
    subnormals m/8 * 2^-6; S.1111.111 is NaN; there is no infinity, so the
    largest finite magnitude is 1.75 * 2^8 = 448.
    """
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6,
                   (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    val = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def decode_e8m0(codes: np.ndarray) -> np.ndarray:
    """OCP E8M0 scale codes (uint8) -> float64: 2^(code-127); 255 is NaN."""
    c = np.asarray(codes).astype(np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))


def dequant_mx32(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MX block-32 dequantisation along the last axis: each run of 32
    e4m3fn elements is multiplied by its own e8m0 scale."""
    v = decode_e4m3fn(codes)
    s = np.repeat(decode_e8m0(scales), 32, axis=-1)
    assert s.shape == v.shape
    return v * s


# ------------------------------------------------------------ cache reading

def cache_rows(data, scale, quantized, page_table_row, positions,
               page_size=64):
    """Rows of one sequence's paged cache at logical ``positions``.

    The physical slot of logical position s is page page_table_row[s // 64],
    row s % 64.  ``data`` is [num_pages, page_size, width]; ``scale`` is
    [num_pages, page_size, width/32] e8m0 codes when ``quantized``.
    Returns float64 [len(positions), width].
    """
    pos = np.asarray(positions, dtype=np.int64)
    page = np.asarray(page_table_row, dtype=np.int64)[pos // page_size]
    slot = pos % page_size
    if quantized:
        return dequant_mx32(data[page, slot], scale[page, slot])
    return decode_bf16(data[page, slot])


# ------------------------------------------------------------------ indexer

def indexer_scores_row(q_idx, w, keys):
    """Lightning Indexer score of one query against candidate keys.

    I[s] = sum_j w[j] * max(0, q_idx[j] . keys[s]) -- per-head dot product,
    ReLU, then the head-weighted sum.  q_idx: [H_I, d_I]; w: [H_I];
    keys: [n, d_I] (one key per position, shared by all indexer heads).
    float64 throughout; exact when the inputs are small integers.
    """
    dots = np.asarray(keys, np.float64) @ np.asarray(q_idx, np.float64).T
    return np.maximum(dots, 0.0) @ np.asarray(w, np.float64)


def topk_row(scores, q_pos, k):
    """Top-K of one score row over the causal candidates 0..q_pos.

    Picks the min(k, q_pos+1) positions with the largest score; equal scores
    go to the lower position first (a stable sort of the negated scores keeps
    ascending position among equals).  Returns int64 [k]: the chosen
    positions in ascending order, then -1 padding.
    """
    n = min(int(q_pos) + 1, len(scores))
    cand = np.asarray(scores[:n], dtype=np.float64)
    order = np.argsort(-cand, kind="stable")
    chosen = np.sort(order[:min(k, n)])
    out = np.full(k, -1, dtype=np.int64)
    out[:len(chosen)] = chosen
    return out


# ---------------------------------------------------------- sparse attention

def sparse_mla_row(q, kv_sel, softmax_scale):
    """Absorbed-MLA attention of one query token over selected latent rows.

    q: [H, 576] (absorbed latent 512 + rope 64 per head); kv_sel: [n, 576]
    (one latent row per selected position, shared by all heads).  Keys are
    the full 576-wide rows, values their first 512 features.
    logit[h, i] = scale * q[h] . kv_sel[i]; softmax over i; out[h] is the
    softmax-weighted sum of values; lse[h] = ln sum_i exp(logit[h, i]).
    An empty selection gives out = 0 and lse = -inf.
    Returns (out float64 [H, 512], lse float64 [H]).
    """
    q = np.asarray(q, np.float64)
    kv_sel = np.asarray(kv_sel, np.float64)
    H = q.shape[0]
    if kv_sel.shape[0] == 0:
        return np.zeros((H, D_VALUE)), np.full(H, -np.inf)
    z = softmax_scale * (q @ kv_sel.T)                  # [H, n]
    m = z.max(axis=1, keepdims=True)
    p = np.exp(z - m)
    l = p.sum(axis=1, keepdims=True)
    out = (p @ kv_sel[:, :D_VALUE]) / l
    lse = (m + np.log(l))[:, 0]
    return out, lse


# ------------------------------------------------------- whole-path drivers

def indexer_scores(inp, rows=None):
    """Scores [B, T, L] (float64) for a contiguous-cache input set; positions
    past a query's position are -inf.  ``rows``: optional list of (b, t) to
    compute (others stay NaN)."""
    wl = inp.wl
    B, T, L = wl.B, wl.T, inp.L
    out = np.full((B, T, L), np.nan)
    want = rows if rows is not None else [(b, t) for b in range(B)
                                          for t in range(T)]
    keys_cache = {}
    for b, t in want:
        if b not in keys_cache:
            keys_cache = {b: cache_rows(inp.k_idx.data, inp.k_idx.scale,
                                        inp.k_idx.quantized,
                                        inp.page_table[b],
                                        np.arange(inp.seq_lens[b]))}
        keys = keys_cache[b]
        qp = int(inp.q_pos[b, t])
        n = min(qp + 1, L)
        row = np.full(L, -np.inf)
        row[:n] = indexer_scores_row(decode_bf16(inp.q_idx[b, t]),
                                     inp.w[b, t], keys[:n])
        out[b, t] = row
    return out


def decode_path(inp, rows=None, want_scores=False):
    """The whole hot path on the CPU: indexer -> Top-K -> sparse attention.

    Reads both caches through the page table.  Returns a dict with idx
    (int64 [B, T, K], -1 padded), out (float64 [B, T, H, 512]) and lse
    (float64 [B, T, H]); rows not requested stay -2 / NaN.  With
    ``want_scores`` also the float64 scores of each requested row.
    """
    wl = inp.wl
    B, T, K, H = wl.B, wl.T, wl.top_k, wl.H
    want = rows if rows is not None else [(b, t) for b in range(B)
                                          for t in range(T)]
    idx = np.full((B, T, K), -2, dtype=np.int64)
    out = np.full((B, T, H, D_VALUE), np.nan)
    lse = np.full((B, T, H), np.nan)
    scores = {}
    cur_b, keys = None, None
    for b, t in want:
        if b != cur_b:
            cur_b = b
            keys = cache_rows(inp.k_idx.data, inp.k_idx.scale,
                              inp.k_idx.quantized, inp.page_table[b],
                              np.arange(inp.seq_lens[b]))
        qp = int(inp.q_pos[b, t])
        n = min(qp + 1, int(inp.seq_lens[b]))
        s = indexer_scores_row(decode_bf16(inp.q_idx[b, t]), inp.w[b, t],
                               keys[:n])
        if want_scores:
            scores[(b, t)] = s
        sel = topk_row(s, qp, K)
        idx[b, t] = sel
        chosen = sel[sel >= 0]
        kv_sel = cache_rows(inp.kv.data, inp.kv.scale, inp.kv.quantized,
                            inp.page_table[b], chosen)
        o, l = sparse_mla_row(decode_bf16(inp.q[b, t]), kv_sel,
                              wl.softmax_scale)
        out[b, t], lse[b, t] = o, l
    res = {"idx": idx, "out": out, "lse": lse}
    if want_scores:
        res["scores"] = scores
    return res
