"""dsa_decode_step_static (the decode step in the library's static device
scratch, for callers that cannot allocate) against dsa_decode_step on the
same inputs: two calls in a row, the second on a smaller input, both
through the C ABI."""
import numpy as np
import pytest
import torch

import indexed_sparse_attention_lightning_amd as dsa
import workloads as wk
from workloads.device import to_device

from gpu_helpers import LSE_ABS_TOL, OUT_REL_TOL, paged_cache

pytestmark = pytest.mark.gpu

W = wk.WORKLOADS


def _both(wl):
    inp = wk.generate(wl)
    d = to_device(inp)
    cache = paged_cache(d)
    msl = int(inp.seq_lens.max())
    qp = d["q_pos"] if wl.T > 1 else None
    shape = (wl.B, wl.T, wl.top_k)
    idx_a = torch.empty(shape, dtype=torch.int32, device="cuda")
    idx_b = torch.empty(shape, dtype=torch.int32, device="cuda")
    out_a, lse_a, _ = dsa.decode_step(cache, d["q_idx"], d["w"], d["q"],
                                      wl.top_k, wl.softmax_scale, msl,
                                      q_pos=qp, idx_out=idx_a)
    out_b, lse_b, _ = dsa.decode_step_static(cache, d["q_idx"], d["w"], d["q"],
                                             wl.top_k, wl.softmax_scale, msl,
                                             q_pos=qp, idx_out=idx_b)
    torch.cuda.synchronize()
    need = dsa.workspace_size(dsa.OP_DECODE_STEP, wl.B, wl.T, msl, wl.H,
                              wl.top_k)
    return need, [x.cpu().numpy()
                  for x in (idx_a, out_a, lse_a, idx_b, out_b, lse_b)]


def test_static_scratch_matches_workspace_entry_point():
    # first the full bf16 decode batch (32 x 32768, 38 MB of scratch), then
    # a smaller paged FP8 batch in the same scratch
    for wl in (W["decode"],
               wk.scaled(W["ragged"], B=3, L_min=100, L_max=3000, top_k=512,
                         seed=104)):
        need, (idx_a, out_a, lse_a, idx_b, out_b, lse_b) = _both(wl)
        assert need <= dsa.STATIC_SCRATCH_BYTES
        assert np.array_equal(idx_a, idx_b), wl.name
        assert np.all(np.isfinite(out_b)) and np.all(np.isfinite(lse_b))
        assert np.abs(out_b - out_a).max() <= OUT_REL_TOL * np.abs(out_a).max()
        assert np.abs(lse_b - lse_a).max() <= LSE_ABS_TOL


def test_static_scratch_rejects_oversized_calls():
    """A call whose workspace would exceed the static scratch is refused
    before any launch."""
    wl = wk.scaled(W["decode"], B=2, L=2048, top_k=256, seed=5)
    inp = wk.generate(wl)
    d = to_device(inp)
    big = 1 << 17   # max_seq_len: B=2 x 131072 scores still fit, so raise B
    assert dsa.workspace_size(dsa.OP_DECODE_STEP, 200, 1, big, wl.H,
                              wl.top_k) > dsa.STATIC_SCRATCH_BYTES
    with pytest.raises(dsa.DsaError, match="WORKSPACE"):
        q_idx = d["q_idx"].repeat(100, 1, 1, 1)
        w = d["w"].repeat(100, 1, 1)
        q = d["q"].repeat(100, 1, 1, 1)
        pt = torch.zeros((200, big // 64), dtype=torch.int32, device="cuda")
        sl = torch.full((200,), 2048, dtype=torch.int32, device="cuda")
        cache = dsa.PagedCache(kidx=d["kidx"], kv=d["kv"], page_table=pt,
                               seq_lens=sl)
        dsa.decode_step_static(cache, q_idx, w, q, wl.top_k, wl.softmax_scale,
                               big)
