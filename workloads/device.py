"""Copy a generated workload to device tensors (torch is plumbing only)."""
from __future__ import annotations

import numpy as np
import torch


def _bf16(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)) \
        .view(torch.bfloat16).to(device)


def _u8(a, device):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_device(inp, device="cuda") -> dict:
    """Device tensors of a ``workloads.Inputs`` in the layouts of the C ABI.

    Keys: q_idx, w, q, q_pos, seq_lens, page_table, kidx, kidx_scale, kv,
    kv_scale (paged pools), and for contiguous inputs kidx_c / kidx_scale_c /
    kv_c / kv_scale_c ([B, L, width] views of the same memory).
    """
    wl = inp.wl
    d = {
        "q_idx": _bf16(inp.q_idx, device),
        "w": torch.from_numpy(inp.w).to(device),
        "q": _bf16(inp.q, device),
        "q_pos": torch.from_numpy(inp.q_pos).to(device),
        "seq_lens": torch.from_numpy(inp.seq_lens).to(device),
        "page_table": torch.from_numpy(inp.page_table).to(device),
    }
    if inp.k_idx.quantized:
        d["kidx"] = _u8(inp.k_idx.data, device)
        d["kidx_scale"] = _u8(inp.k_idx.scale, device)
    else:
        d["kidx"] = _bf16(inp.k_idx.data, device)
        d["kidx_scale"] = None
    if inp.kv.quantized:
        d["kv"] = _u8(inp.kv.data, device)
        d["kv_scale"] = _u8(inp.kv.scale, device)
    else:
        d["kv"] = _bf16(inp.kv.data, device)
        d["kv_scale"] = None
    if inp.contiguous:
        B, L = wl.B, inp.L
        d["kidx_c"] = d["kidx"].view(B, L, wl.d_I)
        d["kv_c"] = d["kv"].view(B, L, 576)
        d["kidx_scale_c"] = None if d["kidx_scale"] is None else \
            d["kidx_scale"].view(B, L, wl.d_I // 32)
        d["kv_scale_c"] = None if d["kv_scale"] is None else \
            d["kv_scale"].view(B, L, 18)
    return d
