"""dsa_decode_step captured in a HIP graph (torch.cuda.CUDAGraph on ROCm).

The step only enqueues kernels on the caller's stream, with all scratch in
the caller's workspace and no memset, so it can be captured.  Each replay,
with eager work and synchronizations between replays, must reproduce the
eager call bit for bit (the kernels are deterministic: integer atomics only,
fixed split and merge order)."""
import pytest
import torch

import indexed_sparse_attention_lightning_amd as dsa
import workloads as wk
from workloads.device import to_device
from gpu_helpers import paged_cache

pytestmark = pytest.mark.gpu

W = wk.WORKLOADS
CASES = {
    "decode_bf16": wk.scaled(W["decode"], B=4, L=4096, top_k=512, seed=21),
    "ragged_fp8": wk.scaled(W["ragged"], B=3, L_min=500, L_max=70000,
                            top_k=1024, seed=22),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_decode_step_graph_replays_match_eager(name):
    wl = CASES[name]
    inp = wk.generate(wl)
    d = to_device(inp)
    cache = paged_cache(d)
    L = int(inp.seq_lens.max())
    ws = torch.empty(dsa.workspace_size(dsa.OP_DECODE_STEP, wl.B, 1, L, wl.H,
                                        wl.top_k), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((wl.B, 1, wl.H, 512), device="cuda")
    lse = torch.empty((wl.B, 1, wl.H), device="cuda")
    idx = torch.empty((wl.B, 1, wl.top_k), dtype=torch.int32, device="cuda")

    def call():
        dsa.decode_step(cache, d["q_idx"], d["w"], d["q"], wl.top_k,
                        wl.softmax_scale, max_seq_len=L, out=out, lse=lse,
                        idx_out=idx, workspace=ws)

    call()
    torch.cuda.synchronize()
    ref = (idx.clone(), out.clone(), lse.clone())

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        idx.fill_(-7)
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[0]), f"replay {rep}: idx differs"
        assert torch.equal(out, ref[1]), f"replay {rep}: out differs"
        assert torch.equal(lse, ref[2]), f"replay {rep}: lse differs"


def test_append_then_decode_graph_replays_match_eager():
    """The decode loop of one layer captured as one graph: store the new
    token's key and latent rows (MX keys, 128-tile KV) with
    dsa_cache_append, then the decode step with the quantised indexer over
    the updated cache.  Every replay rewrites the same slots with the same
    bytes, so each must reproduce the eager pools and outputs bit for bit."""
    wl = wk.scaled(W["decode"], B=3, L=3072, top_k=512, seed=23)
    inp = wk.generate(wl)
    d = to_device(inp)
    B, L = wl.B, int(inp.seq_lens.max())
    P = inp.kv.data.shape[0]
    cache = dsa.PagedCache(
        kidx=torch.zeros((P, 64, wl.d_I), dtype=torch.uint8, device="cuda"),
        kv=torch.zeros((P, 64, 576), dtype=torch.uint8, device="cuda"),
        page_table=d["page_table"], seq_lens=d["seq_lens"],
        kidx_scale=torch.full((P, 64, wl.d_I // 32), 127, dtype=torch.uint8,
                              device="cuda"),
        kv_scale=torch.zeros((P, 64, 5), dtype=torch.float32, device="cuda"))
    # the cache up to the last token, then the last token as the new one
    pos_all = torch.arange(L, dtype=torch.int32, device="cuda").repeat(B, 1)
    pos_all[:, L - 1] = -1
    k_all = d["kidx"].view(P * 64, wl.d_I)[:B * L].view(B, L, wl.d_I)
    v_all = d["kv"].view(P * 64, 576)[:B * L].view(B, L, 576)
    dsa.cache_append(cache, pos_all, k_new=k_all, kv_new=v_all)
    pos_new = torch.full((B, 1), L - 1, dtype=torch.int32, device="cuda")
    k_new = k_all[:, L - 1:].contiguous()
    v_new = v_all[:, L - 1:].contiguous()
    ws = torch.empty(dsa.workspace_size(dsa.OP_DECODE_STEP, B, 1, L, wl.H,
                                        wl.top_k), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((B, 1, wl.H, 512), device="cuda")
    lse = torch.empty((B, 1, wl.H), device="cuda")
    idx = torch.empty((B, 1, wl.top_k), dtype=torch.int32, device="cuda")

    def call():
        dsa.cache_append(cache, pos_new, k_new=k_new, kv_new=v_new)
        dsa.decode_step(cache, d["q_idx"], d["w"], d["q"], wl.top_k,
                        wl.softmax_scale, max_seq_len=L, out=out, lse=lse,
                        idx_out=idx, workspace=ws, quantize_queries=True)

    call()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (idx, out, lse, cache.kidx, cache.kidx_scale,
                               cache.kv, cache.kv_scale)]
    assert torch.isfinite(lse).all()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        idx.fill_(-7)
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        ws.fill_(0xAB)
        # the new token's slots are wiped eagerly: the replay must rewrite them
        for b in range(B):
            pg = int(inp.page_table[b, (L - 1) // 64])
            cache.kv[pg, (L - 1) % 64].fill_(0x7F)
            cache.kv_scale[pg, (L - 1) % 64].fill_(float("nan"))
            cache.kidx[pg, (L - 1) % 64].fill_(0x7F)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (idx, out, lse, cache.kidx, cache.kidx_scale, cache.kv,
               cache.kv_scale)
        for name, a, r in zip(("idx", "out", "lse", "kidx", "kidx_scale",
                               "kv", "kv_scale"), got, ref):
            assert torch.equal(a.view(torch.uint8) if a.dtype == torch.float32
                               else a, r.view(torch.uint8)
                               if r.dtype == torch.float32 else r), \
                f"replay {rep}: {name} differs"
