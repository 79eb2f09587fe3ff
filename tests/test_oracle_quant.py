"""Pins for the oracle's cache quantizers and cache append (CPU only).

The e4m3 rounding is checked against hand-worked values, an exact
brute-force search over all 127 finite magnitudes (rationals, no floating
point), and torch's float8_e4m3fn conversion.  The group and tile scalings
are checked against hand-worked scales, their closed-form inequalities,
round trips of values built from known codes and scales, the input
generator's independent MX quantizer, and tile-boundary probes.  The append
is checked by reading rows back through the (separately pinned) paged-cache
reader.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as wk

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
MAGS = oracle.decode_e4m3fn(np.arange(0x7F))        # finite magnitudes


def _golden():
    return json.load(open(os.path.join(GOLDEN, "hand_quant.json")))


# ---------------------------------------------------------- e4m3 rounding

def test_round_e4m3_hand_golden():
    for what, y, code in _golden()["e4m3_round"]:
        assert int(oracle.round_to_e4m3fn(np.float64(y))) == code, what


def _brute_code(y: float) -> int:
    """Exact nearest finite e4m3fn magnitude by scanning all of them with
    rational arithmetic; ties to the even code; sign from y."""
    a = abs(Fraction(y))
    best, best_d = None, None
    for c in range(0x7F):
        d = abs(Fraction(float(MAGS[c])) - a)
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return best | (0x80 if np.signbit(y) else 0)


def test_round_e4m3_brute_force():
    rng = np.random.default_rng(41)
    mags = np.exp2(rng.uniform(-14, 10, size=600))           # past 448 too
    mids = (MAGS[1:] + MAGS[:-1]) / 2                         # exact ties
    exact = MAGS.copy()
    ys = np.concatenate([mags, mids, exact, -mags[:200], -mids[:60]])
    got = oracle.round_to_e4m3fn(ys)
    for y, c in zip(ys, got):
        assert int(c) == _brute_code(float(y)), y


def test_round_e4m3_vs_torch():
    rng = np.random.default_rng(42)
    x = np.concatenate([
        rng.uniform(-448, 448, 20000),
        np.exp2(rng.uniform(-16, np.log2(448), 20000)) *
        rng.choice([-1.0, 1.0], 20000),
        (MAGS[1:] + MAGS[:-1]) / 2, -(MAGS[1:] + MAGS[:-1]) / 2,
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.round_to_e4m3fn(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_round_e4m3_every_code_is_fixed_point():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F],
                     dtype=np.uint8)
    assert np.array_equal(
        oracle.round_to_e4m3fn(oracle.decode_e4m3fn(codes)), codes)


# ------------------------------------------------------- MX block-32 scale

def test_mx32_scale_hand_golden():
    for what, amax, X in _golden()["mx32_exponent"]:
        row = np.zeros(64)
        row[37] = -amax          # second block; sign must not matter
        codes, sc = oracle.quantize_mx32(row)
        assert int(sc[1]) - 127 == X, what
        assert int(sc[0]) == 127, "an all-zero block takes 2^0"
        if amax > 0:
            # the block maximum maps to its nearest code at that scale
            assert oracle.decode_e4m3fn(codes[37]) * 2.0 ** X <= 0
            assert codes[37] & 0x80


def test_mx32_round_trip_from_codes():
    rng = np.random.default_rng(43)
    n_rows, n_blk = 40, 18
    codes = rng.integers(0, 256, size=(n_rows, n_blk, 32), dtype=np.int64)
    codes[(codes & 0x7F) == 0x7F] = 0x30
    # one element of each block at full scale (|448|), so that the block's
    # exponent is determined by construction
    where = rng.integers(0, 32, size=(n_rows, n_blk))
    sign = rng.integers(0, 2, size=(n_rows, n_blk)) * 0x80
    np.put_along_axis(codes, where[..., None], (0x7E | sign)[..., None], -1)
    X = rng.integers(-100, 100, size=(n_rows, n_blk))
    codes = codes.astype(np.uint8).reshape(n_rows, n_blk * 32)
    x = oracle.dequant_mx32(codes, (X + 127).astype(np.uint8))
    got_c, got_s = oracle.quantize_mx32(x)
    # -0 and +0 codes decode alike; everything else must come back
    assert np.array_equal(got_s.astype(np.int64) - 127, X)
    same = (got_c == codes) | ((got_c & 0x7F) == 0) & ((codes & 0x7F) == 0)
    assert same.all()


def test_mx32_closed_form_error_and_generator_agreement():
    rng = np.random.default_rng(44)
    x = (rng.standard_normal((96, 576)) *
         np.exp(3 * rng.standard_normal((96, 1)))).astype(np.float32)
    x[5, 64:96] = 0.0
    x = wk.f32_to_bf16_bits(x)
    v = oracle.decode_bf16(x)
    codes, sc = oracle.quantize_mx32(v)
    X = sc.astype(np.int64) - 127
    amax = np.abs(v.reshape(96, 18, 32)).max(-1)
    nz = amax > 0
    assert np.all(np.ldexp(448.0, X[nz]) >= amax[nz])
    assert np.all(np.ldexp(448.0, X[nz] - 1) < amax[nz])
    assert sc[5, 2] == 127 and np.all(codes[5, 64:96] == 0)
    back = oracle.dequant_mx32(codes, sc)
    # half a step of a 3-bit mantissa (2^-4 relative), or of the subnormal
    # step 2^-9 * 2^X
    bound = np.abs(v) * 2.0 ** -4 + np.repeat(np.ldexp(2.0 ** -10, X), 32, -1)
    assert np.all(np.abs(back - v) <= bound)
    g_codes, g_sc = wk.mx32_quantize(v.astype(np.float32))
    assert np.array_equal(g_sc, sc)
    assert np.array_equal(g_codes, codes)


# ------------------------------------------------------- tile-128 scale

def test_t128_hand_golden():
    for case in _golden()["t128_tiles"]:
        for tile in range(5):
            lo = oracle.T128_EDGES[tile]
            row = np.zeros(576, dtype=np.float32)
            vals = np.array(case["values"], dtype=np.float32)
            row[lo:lo + len(vals)] = vals
            codes, sc = oracle.quantize_t128(row)
            if "scale" in case:
                assert sc[tile] == np.float32(case["scale"]), case["what"]
            else:
                assert sc[tile] == np.float32(case["scale_num"]) / \
                    np.float32(448.0), case["what"]
            assert codes[lo:lo + len(vals)].tolist() == case["codes"], \
                case["what"]
            others = [i for i in range(5) if i != tile]
            assert np.all(sc[others] == 0)


def test_t128_tile_edges():
    """A large value moves exactly the scale of the tile that holds it."""
    base = np.full(576, 0.5, dtype=np.float32)
    _, s0 = oracle.quantize_t128(base)
    assert np.all(s0 == np.float32(0.5) / np.float32(448))
    edges = oracle.T128_EDGES
    for tile in range(5):
        for pos in (edges[tile], edges[tile + 1] - 1):
            row = base.copy()
            row[pos] = -100.0
            _, s = oracle.quantize_t128(row)
            changed = np.nonzero(s != s0)[0].tolist()
            assert changed == [tile], (pos, changed)
            assert s[tile] == np.float32(100.0) / np.float32(448)


def test_t128_round_trip_power_of_two_scales():
    rng = np.random.default_rng(45)
    rows = 50
    codes = rng.integers(0, 256, size=(rows, 576), dtype=np.int64)
    codes[(codes & 0x7F) == 0x7F] = 0x21
    k = rng.integers(-30, 30, size=(rows, 5))
    for t in range(5):
        lo = oracle.T128_EDGES[t]
        pick = lo + rng.integers(0, oracle.T128_EDGES[t + 1] - lo, size=rows)
        codes[np.arange(rows), pick] = 0x7E | (rng.integers(0, 2, rows) * 0x80)
    codes = codes.astype(np.uint8)
    scales = np.ldexp(1.0, k).astype(np.float32)
    x = oracle.dequant_t128(codes, scales)        # exact in bf16 and fp32
    got_c, got_s = oracle.quantize_t128(x)
    assert np.array_equal(got_s, scales)
    same = (got_c == codes) | ((got_c & 0x7F) == 0) & ((codes & 0x7F) == 0)
    assert same.all()


def test_t128_max_to_448_error_bound_and_torch():
    rng = np.random.default_rng(46)
    v = (rng.standard_normal((64, 576)) *
         np.exp(2 * rng.standard_normal((64, 1)))).astype(np.float32)
    v[7, 128:256] = 0.0
    v[9, 512:] = 0.0
    v = oracle.decode_bf16(wk.f32_to_bf16_bits(v))
    codes, sc = oracle.quantize_t128(v)
    e = oracle.T128_EDGES
    for t in range(5):
        tile = v[:, e[t]:e[t + 1]]
        amax = np.abs(tile).max(-1)
        nz = amax > 0
        assert np.array_equal(sc[:, t],
                              amax.astype(np.float32) / np.float32(448))
        # the element of largest magnitude maps to +-448
        arg = np.abs(tile).argmax(-1)
        top = codes[np.arange(64), e[t] + arg]
        assert np.all((top[nz] & 0x7F) == 0x7E)
    assert np.all(sc[7, 1] == 0) and np.all(sc[9, 4] == 0)
    back = oracle.dequant_t128(codes, sc)
    step = np.repeat(sc.astype(np.float64), np.diff(e), axis=-1)
    bound = np.abs(v) * (2.0 ** -4 + 2.0 ** -20) + step * 2.0 ** -9
    assert np.all(np.abs(back - v) <= bound)
    # torch: the same fp32 divisions, then torch's e4m3fn conversion
    ref = np.empty_like(codes)
    t32 = torch.from_numpy(v.astype(np.float32))
    s32 = torch.from_numpy(sc)
    for t in range(5):
        div = torch.where(s32[:, t] > 0, s32[:, t], torch.ones(()))
        y = (t32[:, e[t]:e[t + 1]] / div[:, None]).clamp(-448, 448)
        ref[:, e[t]:e[t + 1]] = y.to(torch.float8_e4m3fn).view(
            torch.uint8).numpy()
    assert np.array_equal(codes, ref)


def test_dequant_t128_tile_map():
    rng = np.random.default_rng(47)
    codes = rng.integers(0, 256, size=(3, 576), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38
    scales = rng.uniform(0.01, 3, size=(3, 5)).astype(np.float32)
    got = oracle.dequant_t128(codes, scales)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()
    for f in range(576):
        t = min(f // 128, 4)
        assert np.array_equal(got[:, f], ref[:, f] * scales[:, t].astype(
            np.float64))


# ------------------------------------------------------------ cache append

@pytest.mark.parametrize("fmt,width", [("bf16", 576), ("mx32", 576),
                                       ("t128", 576), ("mx32", 128),
                                       ("bf16", 64)])
def test_cache_append_read_back(fmt, width):
    rng = np.random.default_rng(48)
    B, T, max_pages, num_pages = 3, 5, 4, 14
    perm = rng.permutation(num_pages)[:B * max_pages].reshape(B, max_pages)
    page_table = perm.astype(np.int32)
    page_table[2, 3] = -1                     # an unmapped page
    if fmt == "bf16":
        data = rng.integers(0, 1 << 16, size=(num_pages, 64, width)) \
            .astype(np.uint16)
        scale = None
    else:
        data = rng.integers(0, 256, size=(num_pages, 64, width)) \
            .astype(np.uint8)
        scale = (rng.integers(0, 256, size=(num_pages, 64, width // 32))
                 .astype(np.uint8) if fmt == "mx32" else
                 rng.uniform(0, 1, size=(num_pages, 64, 5)).astype(np.float32))
    pos = np.array([[0, 63, 64, 200, 255],
                    [-1, 5, 130, 131, 7],
                    [10, 196, 256, 3, -5]], dtype=np.int32)
    rows = wk.f32_to_bf16_bits(rng.standard_normal((B, T, width))
                               .astype(np.float32))
    rows[0, 1, :32] = 0                        # an all-zero group / tile part
    d0 = data.copy()
    s0 = None if scale is None else scale.copy()
    d1, s1 = oracle.cache_append(data, scale, fmt, page_table, pos, rows)
    written = np.zeros((num_pages, 64), dtype=bool)
    q = {"bf16": False, "mx32": True, "t128": "t128"}[fmt]
    ref = oracle.decode_bf16(rows)
    for b in range(B):
        for t in range(T):
            p = int(pos[b, t])
            if p < 0 or p // 64 >= max_pages or page_table[b, p // 64] < 0:
                continue
            written[page_table[b, p // 64], p % 64] = True
            back = oracle.cache_rows(d1, s1, q, page_table[b], [p])[0]
            if fmt == "bf16":
                assert np.array_equal(back, ref[b, t])
            else:
                step = np.abs(ref[b, t]).max() * 2.0 ** -4 + 1e-30
                assert np.all(np.abs(back - ref[b, t]) <= step)
    assert written.sum() == 11                 # 15 tokens, 4 skipped
    assert np.array_equal(d1[~written], d0[~written])
    if s0 is not None:
        assert np.array_equal(s1[~written], s0[~written])


# ------------------------------------------------ quantised indexer queries

def test_indexer_queries_blocks_are_per_head():
    """Heads of very different magnitude keep their own block scales: every
    element stays within the e4m3 rounding bound of its own block."""
    rng = np.random.default_rng(50)
    q = rng.standard_normal((3, 8, 128)) * \
        np.exp2(rng.integers(-40, 40, size=(3, 8, 1)))
    q[1, 2, 32:64] = 0.0
    bits = wk.f32_to_bf16_bits(q.astype(np.float32))
    v = oracle.decode_bf16(bits)
    got = oracle.indexer_queries(bits, quantize=True)
    blk = np.abs(v).reshape(3, 8, 4, 32).max(-1)
    step = np.repeat(blk, 32, axis=-1) * 2.0 ** -7    # subnormal headroom
    assert np.all(np.abs(got - v) <= np.abs(v) * 2.0 ** -4 + step)
    assert np.all(got[1, 2, 32:64] == 0)
    assert np.array_equal(oracle.indexer_queries(bits), v)


def test_indexer_queries_exact_on_small_integers():
    rng = np.random.default_rng(51)
    bits = wk.f32_to_bf16_bits(
        rng.integers(-4, 5, size=(5, 64, 128)).astype(np.float32))
    assert np.array_equal(oracle.indexer_queries(bits, quantize=True),
                          oracle.decode_bf16(bits))


def _brute_mx_values(row):
    """MX block-32 values of one row by exact search: per block the smallest
    power of two covering max/448, then the nearest code (rationals)."""
    out = []
    for blk in np.asarray(row, dtype=np.float64).reshape(-1, 32):
        amax = Fraction(float(np.abs(blk).max()))
        X = 0
        if amax > 0:
            X = -127
            while Fraction(448) * Fraction(2) ** X < amax:
                X += 1
        scale = Fraction(2) ** X
        for x in blk:
            c = _brute_code(float(Fraction(float(x)) / scale))
            out.append(Fraction(float(oracle.decode_e4m3fn(np.uint8(c)))) * scale)
    return out


def test_quantised_indexer_scores_brute_force():
    wl = wk.WORKLOADS["tiny"]
    inp = wk.generate(wl)
    q = wk.eighths(52, inp.q_idx.shape)
    inp = __import__("dataclasses").replace(inp, q_idx=q)
    got = oracle.indexer_scores(inp, quantize_queries=True)
    keys = oracle.cache_rows(inp.k_idx.data, inp.k_idx.scale,
                             inp.k_idx.quantized, inp.page_table[0],
                             np.arange(inp.seq_lens[0]))
    qv = [_brute_mx_values(oracle.decode_bf16(q[0, 0, j]))
          for j in range(wl.H_I)]
    qp = int(inp.q_pos[0, 0])
    for s in list(range(0, qp + 1, 37)) + [qp]:
        tot = Fraction(0)
        for j in range(wl.H_I):
            d = sum(qv[j][c] * Fraction(float(keys[s, c]))
                    for c in range(wl.d_I))
            tot += Fraction(float(inp.w[0, 0, j])) * max(d, Fraction(0))
        assert got[0, 0, s] == float(tot), s
    # the quantisation changed some query values, so the pin is not vacuous
    assert not np.array_equal(oracle.indexer_queries(q, True),
                              oracle.indexer_queries(q))
