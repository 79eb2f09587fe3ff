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
