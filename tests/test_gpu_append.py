"""Cache append and the 128-tile KV format: HIP path vs CPU oracle (needs an
MI355X).

dsa_cache_append must leave the pools byte-identical to the oracle's append
of the same bf16 rows (codes, e8m0 scale codes and fp32 tile-scale bit
patterns, untouched slots included).  The decode path over a cache built by
the append (MX block-32 indexer keys, 128-tile latent KV) must select the
oracle's indices exactly and match its attention within max|diff| <= 1e-2 *
max|oracle| and |dLSE| <= 1e-3.
"""
import dataclasses

import numpy as np
import pytest
import torch

import indexed_sparse_attention_lightning_amd as dsa
import oracle
import workloads as wk
from workloads.device import to_device

from gpu_helpers import assert_attn_close, assert_idx_equal

pytestmark = pytest.mark.gpu

POISON = {"codes": 0x7F, "e8m0": 0xFF}


def _bf16_t(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)) \
        .view(torch.bfloat16).cuda()


def _pool(rng, fmt, num_pages, width):
    """Random initial pool bytes (data, scale) in the storage of ``fmt``."""
    if fmt == "bf16":
        return rng.integers(0, 1 << 16, size=(num_pages, 64, width)) \
            .astype(np.uint16), None
    data = rng.integers(0, 256, size=(num_pages, 64, width)).astype(np.uint8)
    if fmt == "mx32":
        return data, rng.integers(0, 256, size=(num_pages, 64, width // 32)) \
            .astype(np.uint8)
    return data, rng.standard_normal((num_pages, 64, 5)).astype(np.float32)


def _dev_pool(data, scale):
    d = _bf16_t(data) if data.dtype == np.uint16 else \
        torch.from_numpy(data.copy()).cuda()
    s = None if scale is None else torch.from_numpy(scale.copy()).cuda()
    return d, s


def _same_bytes(got: torch.Tensor, want: np.ndarray, what: str):
    g = got.cpu().contiguous().view(torch.uint8).numpy().reshape(-1)
    w = np.ascontiguousarray(want).view(np.uint8).reshape(-1)
    if not np.array_equal(g, w):
        bad = np.nonzero(g != w)[0]
        raise AssertionError(f"{what}: {len(bad)} bytes differ, first at byte "
                             f"{bad[0]}: got {g[bad[0]]:#x}, want {w[bad[0]]:#x}")


def _append_case(seed, kfmt, vfmt, d_I, B, T, max_pages, extra_pages, pos):
    rng = np.random.default_rng(seed)
    num_pages = B * max_pages + extra_pages
    page_table = rng.permutation(num_pages)[:B * max_pages] \
        .reshape(B, max_pages).astype(np.int32)
    page_table[B - 1, max_pages - 1] = -1                  # unmapped
    page_table[0, max_pages - 1] = num_pages + 3           # outside the pool
    kd, ks = _pool(rng, kfmt, num_pages, d_I)
    vd, vs = _pool(rng, vfmt, num_pages, 576)
    k_rows = wk.append_rows(seed + 1, B * T, d_I).reshape(B, T, d_I)
    v_rows = wk.append_rows(seed + 2, B * T, 576).reshape(B, T, 576)

    dk, dks = _dev_pool(kd, ks)
    dv, dvs = _dev_pool(vd, vs)
    cache = dsa.PagedCache(kidx=dk, kv=dv,
                           page_table=torch.from_numpy(page_table).cuda(),
                           seq_lens=torch.ones(B, dtype=torch.int32).cuda(),
                           kidx_scale=dks, kv_scale=dvs)
    print(f"append case seed={seed} k={kfmt} kv={vfmt} d_I={d_I} B={B} T={T}",
          flush=True)
    dsa.cache_append(cache, torch.from_numpy(pos).cuda(),
                     k_new=_bf16_t(k_rows), kv_new=_bf16_t(v_rows))
    torch.cuda.synchronize()

    ok_, oks = oracle.cache_append(kd.copy(), None if ks is None else ks.copy(),
                                   kfmt, page_table, pos, k_rows)
    ov, ovs = oracle.cache_append(vd.copy(), None if vs is None else vs.copy(),
                                  vfmt, page_table, pos, v_rows)
    _same_bytes(dk, ok_, "indexer-key pool")
    _same_bytes(dv, ov, "latent pool")
    if ks is not None:
        _same_bytes(dks, oks, "indexer-key scales")
    if vs is not None:
        _same_bytes(dvs, ovs, "latent scales")
    # the case must write something and skip something
    assert not np.array_equal(ov, vd)


def _positions(rng, B, T, max_pages):
    """Unique positions per sequence, with skipped tokens of every kind."""
    pos = np.stack([rng.permutation(max_pages * 64)[:T] for _ in range(B)]) \
        .astype(np.int32)
    pos[0, 0] = -1
    pos[min(1, B - 1), -1] = max_pages * 64 + 5     # past the page table
    pos[0, 1] = (max_pages - 1) * 64 + 7            # page entry outside pool
    pos[B - 1, 2] = (max_pages - 1) * 64            # unmapped page
    return pos


@pytest.mark.parametrize("kfmt,vfmt,d_I", [
    ("bf16", "bf16", 128), ("mx32", "mx32", 128), ("mx32", "t128", 128),
    ("bf16", "t128", 64), ("mx32", "bf16", 64)])
def test_append_matches_oracle(kfmt, vfmt, d_I):
    rng = np.random.default_rng(200)
    B, T, max_pages = 3, 40, 3
    pos = _positions(rng, B, T, max_pages)
    _append_case(201, kfmt, vfmt, d_I, B, T, max_pages, 5, pos)


def test_append_many_tokens_ragged_grid():
    """903 tokens: the last workgroup holds fewer than four."""
    rng = np.random.default_rng(210)
    B, T, max_pages = 3, 301, 6
    pos = _positions(rng, B, T, max_pages)
    _append_case(211, "mx32", "t128", 128, B, T, max_pages, 2, pos)


def test_append_one_token():
    pos = np.array([[130]], dtype=np.int32)
    _append_case(220, "mx32", "mx32", 128, 1, 1, 4, 0, pos)


# ----------------------------------------------- decode over appended caches

def _appended_cache(inp, kfmt="mx32", vfmt="t128"):
    """Quantised pools built from a bf16 workload's rows: on the device by
    dsa.cache_append, on the host by the oracle.  Returns (device cache,
    oracle inputs over the host pools)."""
    wl = inp.wl
    assert not inp.k_idx.quantized and not inp.kv.quantized
    B = wl.B
    lens = inp.seq_lens.astype(np.int64)
    Lmax = int(lens.max())
    num_pages = inp.kv.data.shape[0]
    pos = np.where(np.arange(Lmax)[None, :] < lens[:, None],
                   np.arange(Lmax)[None, :], -1).astype(np.int32)
    safe = np.maximum(pos, 0)
    pages = inp.page_table[np.arange(B)[:, None], safe // 64]
    k_rows = inp.k_idx.data[pages, safe % 64]            # [B, Lmax, d_I]
    v_rows = inp.kv.data[pages, safe % 64]               # [B, Lmax, 576]
    k_rows[pos < 0] = 0
    v_rows[pos < 0] = 0

    def empty(fmt, width):
        data = np.full((num_pages, 64, width), POISON["codes"], np.uint8)
        if fmt == "mx32":
            return data, np.full((num_pages, 64, width // 32), POISON["e8m0"],
                                 np.uint8)
        return data, np.full((num_pages, 64, 5), np.nan, np.float32)

    kd, ks = empty(kfmt, wl.d_I)
    vd, vs = empty(vfmt, 576)
    d = to_device(inp)
    dk, dks = _dev_pool(kd, ks)
    dv, dvs = _dev_pool(vd, vs)
    cache = dsa.PagedCache(kidx=dk, kv=dv, page_table=d["page_table"],
                           seq_lens=d["seq_lens"], kidx_scale=dks,
                           kv_scale=dvs)
    dsa.cache_append(cache, torch.from_numpy(pos).cuda(),
                     k_new=_bf16_t(k_rows), kv_new=_bf16_t(v_rows))
    torch.cuda.synchronize()
    oracle.cache_append(kd, ks, kfmt, inp.page_table, pos, k_rows)
    oracle.cache_append(vd, vs, vfmt, inp.page_table, pos, v_rows)
    _same_bytes(dk, kd, "appended key pool")
    _same_bytes(dv, vd, "appended latent pool")
    _same_bytes(dks, ks, "appended key scales")
    _same_bytes(dvs, vs, "appended latent scales")
    q = {"bf16": False, "mx32": True, "t128": "t128"}
    ref_inp = dataclasses.replace(
        inp, k_idx=wk.Cache(kd, ks, q[kfmt]), kv=wk.Cache(vd, vs, q[vfmt]))
    return d, cache, ref_inp


T128_CASES = {
    "decode_t128": wk.scaled(wk.WORKLOADS["decode"], B=3, L=2048, top_k=256,
                             seed=301),
    "ragged_t128": wk.scaled(wk.WORKLOADS["ragged"], B=3, L_min=200,
                             L_max=3000, top_k=512, quantized=False, seed=302),
    "prefill_t128": wk.scaled(wk.WORKLOADS["prefill"], T=33, L=1280,
                              first_pos=1200, top_k=384, H=32, seed=303),
}


@pytest.mark.parametrize("name", sorted(T128_CASES))
def test_decode_over_appended_t128_cache(name):
    wl = T128_CASES[name]
    inp = wk.generate(wl)
    print(f"t128 decode case {name}", flush=True)
    d, cache, ref_inp = _appended_cache(inp)
    rows = [(b, t) for b in range(wl.B) for t in range(wl.T)]
    ref = oracle.decode_path(ref_inp, rows=rows)
    idx = torch.empty((wl.B, wl.T, wl.top_k), dtype=torch.int32, device="cuda")
    out, lse, _ = dsa.decode_step(
        cache, d["q_idx"], d["w"], d["q"], wl.top_k, wl.softmax_scale,
        max_seq_len=int(inp.seq_lens.max()),
        q_pos=d["q_pos"] if wl.T > 1 else None, idx_out=idx)
    torch.cuda.synchronize()
    assert_idx_equal(idx.cpu().numpy(), ref["idx"], rows)
    assert_attn_close(out.cpu().numpy(), lse.cpu().numpy(), ref, rows)
    if inp.contiguous:
        # the separate attention entry point over the contiguous view
        B, L = wl.B, inp.L
        out2, lse2 = dsa.sparse_mla_attn(
            d["q"], cache.kv.view(B, L, 576), idx, wl.softmax_scale,
            kv_scale=cache.kv_scale.view(B, L, 5))
        torch.cuda.synchronize()
        assert_attn_close(out2.cpu().numpy(), lse2.cpu().numpy(), ref, rows)


@pytest.mark.parametrize("which", ["keys_only", "latent_only"])
def test_append_one_pool(which):
    """Appending only one pool leaves the other untouched."""
    rng = np.random.default_rng(230)
    B, T, max_pages, num_pages = 2, 9, 2, 4
    page_table = np.array([[0, 2], [1, 3]], dtype=np.int32)
    kd, ks = _pool(rng, "mx32", num_pages, 128)
    vd, vs = _pool(rng, "t128", num_pages, 576)
    pos = np.stack([rng.permutation(128)[:T] for _ in range(B)]).astype(np.int32)
    k_rows = wk.append_rows(231, B * T, 128).reshape(B, T, 128)
    v_rows = wk.append_rows(232, B * T, 576).reshape(B, T, 576)
    dk, dks = _dev_pool(kd, ks)
    dv, dvs = _dev_pool(vd, vs)
    cache = dsa.PagedCache(kidx=dk, kv=dv,
                           page_table=torch.from_numpy(page_table).cuda(),
                           seq_lens=torch.ones(B, dtype=torch.int32).cuda(),
                           kidx_scale=dks, kv_scale=dvs)
    keys = which == "keys_only"
    dsa.cache_append(cache, torch.from_numpy(pos).cuda(),
                     k_new=_bf16_t(k_rows) if keys else None,
                     kv_new=None if keys else _bf16_t(v_rows))
    torch.cuda.synchronize()
    if keys:
        ok_, oks = oracle.cache_append(kd.copy(), ks.copy(), "mx32",
                                       page_table, pos, k_rows)
        _same_bytes(dk, ok_, "key pool")
        _same_bytes(dks, oks, "key scales")
        _same_bytes(dv, vd, "latent pool (untouched)")
        _same_bytes(dvs, vs, "latent scales (untouched)")
    else:
        ov, ovs = oracle.cache_append(vd.copy(), vs.copy(), "t128",
                                      page_table, pos, v_rows)
        _same_bytes(dv, ov, "latent pool")
        _same_bytes(dvs, ovs, "latent scales")
        _same_bytes(dk, kd, "key pool (untouched)")
        _same_bytes(dks, ks, "key scales (untouched)")
