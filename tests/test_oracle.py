"""Pins for the CPU oracle (CPU only).

Each test checks the oracle against something other than itself: pure-Python
brute force over exact rationals, torch's own bf16/fp8 decoders, torch's dense
scaled-dot-product attention, hand-worked fixtures under tests/golden/,
closed forms and invariants.  Together they are chosen so that a dropped term,
a wrong sign or index, or a transposed operand in the oracle fails at least
one of them.
"""
import dataclasses
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as wk

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------ decoding pins

def test_bf16_decode_all_patterns_vs_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16) \
        .to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e4m3fn_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e8m0_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_e8m0(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu) \
        .to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_fp8_hand_values_golden():
    g = json.load(open(os.path.join(GOLDEN, "hand_fp8.json")))
    for code, val in g["e4m3"]:
        got = oracle.decode_e4m3fn(np.uint8(code))
        assert got == val and np.signbit(got) == np.signbit(val), code
    for code in g["e4m3_nan"]:
        assert np.isnan(oracle.decode_e4m3fn(np.uint8(code)))
    for code, val in g["e8m0"]:
        assert oracle.decode_e8m0(np.uint8(code)) == val, code
    for code in g["e8m0_nan"]:
        assert np.isnan(oracle.decode_e8m0(np.uint8(code)))


def test_dequant_mx32_block_structure():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, size=(3, 96), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38
    scales = np.array([[120, 127, 130], [127, 127, 127], [100, 140, 127]],
                      dtype=np.uint8)
    got = oracle.dequant_mx32(codes, scales)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()
    for r in range(3):
        for blk in range(3):
            sl = slice(32 * blk, 32 * blk + 32)
            assert np.array_equal(got[r, sl],
                                  ref[r, sl] * 2.0 ** (int(scales[r, blk]) - 127))


# ------------------------------------------------------------ indexer pins

def _brute_scores(q_idx, w, keys, q_pos):
    """Exact rational scores by Python loops (ints and Fractions)."""
    out = []
    for s in range(q_pos + 1):
        tot = Fraction(0)
        for j in range(len(q_idx)):
            d = sum(int(a) * int(b) for a, b in zip(q_idx[j], keys[s]))
            tot += Fraction(w[j]) * max(0, d)
        out.append(tot)
    return out


def _brute_topk(scores, k):
    order = sorted(range(len(scores)), key=lambda s: (-scores[s], s))[:k]
    chosen = sorted(order)
    return chosen + [-1] * (k - len(chosen))


@pytest.mark.parametrize("seed", range(12))
def test_indexer_and_topk_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    H_I = int(rng.integers(1, 4))
    d_I = int(rng.integers(1, 5))
    L = int(rng.integers(1, 48))
    q_pos = int(rng.integers(0, L))
    k = int(rng.integers(1, 20))
    q_idx = rng.integers(-2, 3, size=(H_I, d_I))
    keys = rng.integers(-2, 3, size=(L, d_I))
    w = [2.0 ** -int(u) for u in rng.integers(0, 4, size=H_I)]
    exact = _brute_scores(q_idx, w, keys, q_pos)
    got = oracle.indexer_scores_row(q_idx, np.array(w), keys[:q_pos + 1])
    assert [Fraction(float(x)) for x in got] == exact
    want = _brute_topk(exact, k)
    assert oracle.topk_row(got, q_pos, k).tolist() == want
    # a full-length score row with junk past q_pos must give the same picks
    padded = np.concatenate([got, np.full(L - q_pos - 1, 1e9)])
    assert oracle.topk_row(padded, q_pos, k).tolist() == want


def test_topk_hand_golden():
    g = json.load(open(os.path.join(GOLDEN, "hand_topk.json")))
    for case in g["cases"]:
        keys = np.array(case["keys"], dtype=np.float64)
        n = case["q_pos"] + 1
        s = oracle.indexer_scores_row(np.array(case["q_idx"], np.float64),
                                      np.array(case["w"]), keys[:n])
        assert s.tolist() == case["scores"], case["name"]
        got = oracle.topk_row(s, case["q_pos"], case["k"])
        assert got.tolist() == case["idx"], case["name"]


def test_indexer_integer_exactness():
    """8*I is an integer for integer q/k and w = 2^-u; an int64 computation
    of it must equal the float64 oracle exactly."""
    rng = np.random.default_rng(7)
    H_I, d_I, L = 64, 128, 777
    q = rng.integers(-4, 5, size=(H_I, d_I))
    keys = rng.integers(-4, 5, size=(L, d_I))
    u = rng.integers(0, 4, size=H_I)
    dots = keys.astype(np.int64) @ q.T.astype(np.int64)
    eight_i = np.maximum(dots, 0) @ (8 >> u).astype(np.int64)
    got = oracle.indexer_scores_row(q, np.ldexp(1.0, -u), keys)
    assert np.array_equal(got * 8, eight_i.astype(np.float64))
    assert eight_i.max() < 2 ** 24     # also exact in float32


def test_topk_all_zero_query():
    keys = np.random.default_rng(3).integers(-4, 5, size=(300, 16))
    s = oracle.indexer_scores_row(np.zeros((4, 16)), np.ones(4), keys)
    assert np.all(s == 0)
    assert oracle.topk_row(s, 299, 50).tolist() == list(range(50))


# --------------------------------------------------- sparse attention pins

def _sdpa_dense(q, kv, scale):
    """Dense attention over all rows via torch (float64, CPU)."""
    H = q.shape[0]
    qt = torch.from_numpy(q).reshape(1, H, 1, 576)
    kt = torch.from_numpy(kv).reshape(1, 1, -1, 576).expand(1, H, -1, 576)
    vt = torch.from_numpy(np.ascontiguousarray(kv[:, :512])) \
        .reshape(1, 1, -1, 512).expand(1, H, -1, 512)
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.contiguous(), vt.contiguous(), scale=scale)
    logits = scale * (torch.from_numpy(q) @ torch.from_numpy(kv).T)
    return out.reshape(H, 512).numpy(), torch.logsumexp(logits, 1).numpy()


def test_sparse_mla_dense_reduction_via_full_path():
    """Top-K with k >= history length reproduces dense MLA attention."""
    wl = wk.scaled(wk.WORKLOADS["tiny"], L=128, top_k=200, H=8, seed=11)
    inp = wk.generate(wl)
    res = oracle.decode_path(inp)
    q = oracle.decode_bf16(inp.q[0, 0])
    kv = oracle.decode_bf16(inp.kv.data.reshape(-1, 576)[:128])
    ref_out, ref_lse = _sdpa_dense(q, kv, wl.softmax_scale)
    assert res["idx"][0, 0].tolist() == list(range(128)) + [-1] * 72
    np.testing.assert_allclose(res["out"][0, 0], ref_out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(res["lse"][0, 0], ref_lse, rtol=0, atol=1e-12)


def test_sparse_mla_closed_form_two_rows():
    """Two selected rows: softmax weights are a logistic of the logit gap."""
    scale = 1 / math.sqrt(192)
    q = np.zeros((2, 576))
    q[0, 0], q[1, 513] = 3.0, -2.0
    kv = np.zeros((2, 576))
    kv[0, 0], kv[1, 0] = 1.0, -1.0
    kv[0, 513], kv[1, 513] = 0.5, 2.0
    kv[0, 7], kv[1, 7] = 10.0, 20.0        # a value-only feature
    out, lse = oracle.sparse_mla_row(q, kv, scale)
    for h, (z0, z1) in enumerate([(3.0 * scale, -3.0 * scale),
                                  (-1.0 * scale, -4.0 * scale)]):
        p0 = 1.0 / (1.0 + math.exp(z1 - z0))
        assert abs(out[h, 0] - (p0 * 1.0 + (1 - p0) * -1.0)) < 1e-14
        assert abs(out[h, 7] - (p0 * 10.0 + (1 - p0) * 20.0)) < 1e-13
        assert abs(lse[h] - math.log(math.exp(z0) + math.exp(z1))) < 1e-14
    # the rope features (512..575) score but never appear in the output
    assert out.shape == (2, 512)


def test_sparse_mla_invariants():
    rng = np.random.default_rng(9)
    H, n, scale = 6, 40, 1 / math.sqrt(192)
    q = rng.standard_normal((H, 576))
    kv = rng.standard_normal((n, 576))
    out, lse = oracle.sparse_mla_row(q, kv, scale)
    perm = rng.permutation(n)
    out_p, lse_p = oracle.sparse_mla_row(q, kv[perm], scale)
    np.testing.assert_allclose(out_p, out, atol=1e-13)
    np.testing.assert_allclose(lse_p, lse, atol=1e-13)
    z = scale * q @ kv.T
    assert np.all(z.max(1) <= lse + 1e-12)
    assert np.all(lse <= z.max(1) + math.log(n) + 1e-12)
    vmin, vmax = kv[:, :512].min(0), kv[:, :512].max(0)
    assert np.all(out >= vmin - 1e-12) and np.all(out <= vmax + 1e-12)
    const = np.tile(rng.standard_normal(576), (n, 1))
    oc, _ = oracle.sparse_mla_row(q, const, scale)
    np.testing.assert_allclose(oc, np.tile(const[0, :512], (H, 1)), atol=1e-13)
    oe, le = oracle.sparse_mla_row(q, kv[:0], scale)
    assert np.all(oe == 0) and np.all(np.isneginf(le))


# ------------------------------------------------------- whole-path pins

def _small(name, **kw):
    return wk.scaled(wk.WORKLOADS[name], **kw)


def test_causality_and_counts():
    wl = _small("prefill", T=9, L=640, first_pos=300, top_k=128, H=4, H_I=4,
                d_I=32, seed=21)
    inp = wk.generate(wl)
    res = oracle.decode_path(inp)
    for t in range(wl.T):
        row = res["idx"][0, t]
        qp = int(inp.q_pos[0, t])
        sel = row[row >= 0]
        assert len(sel) == min(wl.top_k, qp + 1)
        assert np.all(sel <= qp) and len(set(sel.tolist())) == len(sel)
        assert np.all(np.diff(sel) > 0) and np.all(row[len(sel):] == -1)


def test_paged_equals_contiguous():
    """Reading through a random page table gives the contiguous result."""
    wl = _small("ragged", B=3, L_min=150, L_max=700, top_k=96, H=4, H_I=8,
                d_I=64, seed=31)
    inp = wk.generate(wl)
    assert (inp.k_idx.data.shape[0] == inp.page_table.max() + 1)
    res = oracle.decode_path(inp)
    # undo the scatter: sequence b's pages gathered into logical order
    for b in range(wl.B):
        n = int(inp.seq_lens[b])
        npg = -(-n // 64)
        pages = inp.page_table[b, :npg]
        kd = inp.k_idx.data[pages].reshape(-1, wl.d_I)[:n]
        ks = inp.k_idx.scale[pages].reshape(-1, wl.d_I // 32)[:n]
        vd = inp.kv.data[pages].reshape(-1, 576)[:n]
        vs = inp.kv.scale[pages].reshape(-1, 18)[:n]
        keys = oracle.dequant_mx32(kd, ks)
        s = oracle.indexer_scores_row(oracle.decode_bf16(inp.q_idx[b, 0]),
                                      inp.w[b, 0], keys)
        sel = oracle.topk_row(s, n - 1, wl.top_k)
        assert np.array_equal(sel, res["idx"][b, 0])
        o, l = oracle.sparse_mla_row(oracle.decode_bf16(inp.q[b, 0]),
                                     oracle.dequant_mx32(vd, vs)[sel[sel >= 0]],
                                     wl.softmax_scale)
        np.testing.assert_array_equal(o, res["out"][b, 0])
        np.testing.assert_array_equal(l, res["lse"][b, 0])


def test_fp8_keys_select_the_same_positions():
    """Integer keys in [-4, 4] survive MX quantisation exactly, so the FP8
    path selects exactly the bf16 path's positions."""
    kw = dict(B=2, L=1024, top_k=128, H=4)
    a = wk.generate(_small("decode", **kw))
    b = wk.generate(_small("decode_fp8", **kw))
    ra, rb = oracle.decode_path(a), oracle.decode_path(b)
    assert np.array_equal(ra["idx"], rb["idx"])
    # MXFP8 latent KV: e4m3 keeps 3 mantissa bits, so outputs move a little
    assert np.max(np.abs(ra["out"] - rb["out"])) < 0.2


def test_scores_api_shape_and_mask():
    wl = _small("prefill", T=5, L=256, first_pos=100, top_k=32, H=2, H_I=2,
                d_I=64, seed=41)
    inp = wk.generate(wl)
    sc = oracle.indexer_scores(inp)
    for t in range(5):
        qp = 100 + t
        assert np.all(np.isneginf(sc[0, t, qp + 1:]))
        assert np.all(np.isfinite(sc[0, t, :qp + 1]))
        assert np.all(sc[0, t, :qp + 1] >= 0)


# ---------------------------------------------------- generator sanity

def test_mx_quantizer_scale_rule_and_error():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 576)).astype(np.float32) * \
        np.exp(rng.standard_normal((64, 1))).astype(np.float32)
    x[3, 32:64] = 0.0
    codes, sc = wk.mx32_quantize(x)
    X = sc.astype(np.int64) - 127
    amax = np.abs(x.reshape(64, 18, 32)).max(-1).astype(np.float64)
    nz = amax > 0
    assert np.all(np.ldexp(448.0, X[nz]) >= amax[nz])
    assert np.all(np.ldexp(448.0, X[nz] - 1) < amax[nz])
    assert sc[3, 1] == 127 and np.all(codes[3, 32:64] == 0)
    back = oracle.dequant_mx32(codes, sc)
    err = np.abs(back - x)
    # RNE to 3 mantissa bits: relative error <= 2^-4 for normals, plus the
    # subnormal step 2^-9 * scale
    bound = np.abs(x) * 2.0 ** -4 + np.repeat(np.ldexp(2.0 ** -10, X), 32, -1)
    assert np.all(err <= bound)


def test_generator_deterministic_and_shapes():
    a = wk.generate(wk.WORKLOADS["tiny"])
    b = wk.generate(wk.WORKLOADS["tiny"])
    for f in ("q_idx", "w", "q", "q_pos", "page_table"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    assert np.array_equal(a.kv.data, b.kv.data)
    assert a.q_idx.shape == (1, 1, 4, 64) and a.q.shape == (1, 1, 16, 576)
    assert a.k_idx.data.shape == (8, 64, 64) and a.kv.data.shape == (8, 64, 576)
    assert a.q_pos.tolist() == [[511]]
    qi = oracle.decode_bf16(a.q_idx)
    assert set(np.unique(qi).tolist()) <= set(range(-3, 4))
    assert set(np.unique(a.w).tolist()) <= {1.0, 0.5, 0.25, 0.125}


def test_ragged_tail_is_poisoned():
    wl = _small("ragged", B=2, L_min=100, L_max=200, H=2, H_I=4, d_I=64,
                top_k=16, seed=4)
    inp = wk.generate(wl)
    for b in range(2):
        n = int(inp.seq_lens[b])
        last = inp.page_table[b, (n - 1) // 64]
        tail = inp.kv.data[last, n % 64:] if n % 64 else inp.kv.data[last, :0]
        assert np.all(tail == wk.E4M3_NAN_CODE)
