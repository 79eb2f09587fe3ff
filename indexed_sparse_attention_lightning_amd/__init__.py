"""Indexed sparse attention (DSA) hot path for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI in ``include/dsa.h`` (``libdsa.so``, built
in-tree by ``python -m indexed_sparse_attention_lightning_amd.build``).  The
binding only marshals arguments: PyTorch provides device memory and the
current HIP stream; every step of the path runs in the library's kernels.
There is no fallback: if the library is missing or fails to load, importing
this package raises.

Entry points (same names as the C ABI, without the ``dsa_`` prefix):

* ``indexer_scores``  Lightning Indexer scores over a contiguous key cache
* ``topk``            per-row Top-K (ties to the lower position), ascending
* ``sparse_mla_attn`` absorbed-MLA attention over selected latent rows
* ``decode_step``     indexer -> Top-K -> attention over a paged cache
* ``decode_step_static``  the same in the library's static device scratch
                      (no workspace: for callers that cannot allocate)
* ``indexer_topk``    indexer and Top-K in one kernel over the paged keys
                      (scores kept on chip; rows up to 32768 positions)
* ``cache_append``    store new tokens' key / latent rows into the paged
                      pools, quantised to each pool's format
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

__all__ = [
    "DSA_BF16", "DSA_E4M3_MX32", "DSA_E4M3_T128", "DSA_Q_BF16", "DSA_Q_MX32",
    "DsaError", "PagedCache",
    "cache_append", "decode_step", "decode_step_static", "indexer_scores",
    "indexer_topk", "library_path", "FUSED_MAX_CONTEXT", "STATIC_SCRATCH_BYTES",
    "sparse_mla_attn", "topk", "workspace_size",
]

DSA_BF16 = 0
DSA_E4M3_MX32 = 1
DSA_E4M3_T128 = 2
T128_TILES = 5
DSA_Q_BF16, DSA_Q_MX32 = 0, 1
OP_INDEXER_SCORES, OP_TOPK, OP_SPARSE_MLA, OP_DECODE_STEP = 0, 1, 2, 3
LATENT, VALUE, PAGE = 576, 512, 64
STATIC_SCRATCH_BYTES = 64 << 20   # DSA_STATIC_SCRATCH_BYTES
FUSED_MAX_CONTEXT = 32768         # DSA_FUSED_MAX_CONTEXT

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdsa.so")


class DsaError(RuntimeError):
    """A non-zero dsa_status from the library."""


class _PagedCacheC(ctypes.Structure):
    _fields_ = [
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("kidx_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("kidx", ctypes.c_void_p),
        ("kidx_scale", ctypes.c_void_p),
        ("kv", ctypes.c_void_p),
        ("kv_scale", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
    ]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with "
            "`python -m indexed_sparse_attention_lightning_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    I, P, F, S = ctypes.c_int, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
    sig = {
        "dsa_indexer_scores": [I, I, I, I, I, P, I, P, P, I, P, P, P, P],
        "dsa_topk": [I, I, I, I, P, P, P, P, S, P],
        "dsa_sparse_mla_attn": [I, I, I, I, I, P, P, I, P, P, F, P, P, P, S, P],
        "dsa_decode_step": [I, I, I, I, I, I, F, ctypes.POINTER(_PagedCacheC),
                            I, P, I, P, P, P, P, P, P, P, S, P],
        "dsa_decode_step_static": [I, I, I, I, I, I, F,
                                   ctypes.POINTER(_PagedCacheC),
                                   I, P, I, P, P, P, P, P, P, P],
        "dsa_indexer_topk": [I, I, I, I, I, ctypes.POINTER(_PagedCacheC), I,
                             P, I, P, P, P, P],
        "dsa_cache_append": [I, I, I, I, I, P, P, P, I, P, P, P, I, P, P, P],
        "dsa_workspace_size": [I, I, I, I, I, I],
        "dsa_status_string": [I],
        "dsa_last_error": [],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
    for name in ("dsa_indexer_scores", "dsa_topk", "dsa_sparse_mla_attn",
                 "dsa_decode_step", "dsa_decode_step_static",
                 "dsa_indexer_topk", "dsa_cache_append"):
        getattr(lib, name).restype = ctypes.c_int
    lib.dsa_workspace_size.restype = ctypes.c_size_t
    lib.dsa_status_string.restype = ctypes.c_char_p
    lib.dsa_last_error.restype = ctypes.c_char_p
    return lib


_lib = _load()


def library_path() -> str:
    return _LIB_PATH


def _check(status: int, what: str) -> None:
    if status != 0:
        msg = _lib.dsa_last_error().decode()
        kind = _lib.dsa_status_string(status).decode()
        raise DsaError(f"{what}: {kind}: {msg}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _need(t: torch.Tensor, name: str, dtype, shape=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, "
                         f"got {tuple(t.shape)}")


def workspace_size(op: int, B: int, T: int, L: int, H: int, K: int) -> int:
    return int(_lib.dsa_workspace_size(op, B, T, L, H, K))


def _cache_dtype(t: torch.Tensor, scale: Optional[torch.Tensor], name: str,
                 tiles_ok: bool = False):
    """Storage format of a cache tensor: bf16 values; uint8 e4m3 codes with
    uint8 e8m0 group scales (MX32); or, for latent KV, uint8 codes with
    float32 tile scales (T128)."""
    if t.dtype == torch.bfloat16:
        if scale is not None:
            raise ValueError(f"{name}: bf16 cache takes no scales")
        return DSA_BF16
    if t.dtype == torch.uint8:
        if scale is None:
            raise ValueError(f"{name}: e4m3 codes need scales")
        if scale.dtype == torch.uint8:
            return DSA_E4M3_MX32
        if scale.dtype == torch.float32 and tiles_ok:
            return DSA_E4M3_T128
        raise TypeError(f"{name}: scales must be uint8 e8m0"
                        + (" or float32 tile scales" if tiles_ok else ""))
    raise TypeError(f"{name} must be bfloat16 or uint8 (e4m3 codes)")


def _scale_shape(dtype: int, lead, width: int):
    return (*lead, T128_TILES) if dtype == DSA_E4M3_T128 else \
        (*lead, width // 32)


def indexer_scores(q_idx: torch.Tensor, w: torch.Tensor, k_idx: torch.Tensor,
                   q_pos: torch.Tensor, k_scale: Optional[torch.Tensor] = None,
                   out: Optional[torch.Tensor] = None,
                   quantize_queries: bool = False) -> torch.Tensor:
    """Scores [B, T, L] fp32: sum_j w[t,j] * relu(q_I[t,j] . k_I[s]) for
    s <= q_pos, -inf beyond.  k_idx: [B, L, d_I] bf16, or uint8 e4m3 codes
    with k_scale [B, L, d_I/32] uint8 e8m0.  quantize_queries: the fully
    quantised indexer (queries to MX block-32 on the fly, scaled FP8 matrix
    cores; MX keys only)."""
    B, T, H_I, d_I = q_idx.shape
    L = k_idx.shape[1]
    _need(q_idx, "q_idx", torch.bfloat16)
    _need(w, "w", torch.float32, (B, T, H_I))
    _need(q_pos, "q_pos", torch.int32, (B, T))
    kd = _cache_dtype(k_idx, k_scale, "k_idx")
    _need(k_idx, "k_idx", k_idx.dtype, (B, L, d_I))
    if k_scale is not None:
        _need(k_scale, "k_scale", torch.uint8, (B, L, d_I // 32))
    if out is None:
        out = torch.empty((B, T, L), dtype=torch.float32, device=q_idx.device)
    _need(out, "scores", torch.float32, (B, T, L))
    _check(_lib.dsa_indexer_scores(B, T, L, H_I, d_I, _ptr(q_idx),
                                   DSA_Q_MX32 if quantize_queries else
                                   DSA_Q_BF16, _ptr(w),
                                   _ptr(k_idx), kd, _ptr(k_scale),
                                   _ptr(q_pos), _ptr(out), _stream()),
           "dsa_indexer_scores")
    return out


def topk(scores: torch.Tensor, q_pos: torch.Tensor, k: int,
         out: Optional[torch.Tensor] = None,
         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """idx [B, T, k] int32: the min(k, q_pos+1) best positions of each row
    (ties to the lower position), ascending, then -1.  Rows longer than
    65536 use a workspace of workspace_size(OP_TOPK, ...) bytes (allocated
    here when not given; an empty tensor selects the one-workgroup path)."""
    B, T, L = scores.shape
    _need(scores, "scores", torch.float32)
    _need(q_pos, "q_pos", torch.int32, (B, T))
    if out is None:
        out = torch.empty((B, T, k), dtype=torch.int32, device=scores.device)
    _need(out, "idx", torch.int32, (B, T, k))
    if workspace is None:
        ws_bytes = workspace_size(OP_TOPK, B, T, L, 1, k)
        if ws_bytes:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8,
                                    device=scores.device)
    _check(_lib.dsa_topk(B, T, L, k, _ptr(scores), _ptr(q_pos), _ptr(out),
                         _ptr(workspace) if workspace is not None and
                         workspace.numel() else None,
                         0 if workspace is None else workspace.numel(),
                         _stream()), "dsa_topk")
    return out


def sparse_mla_attn(q: torch.Tensor, kv: torch.Tensor, idx: torch.Tensor,
                    softmax_scale: float,
                    kv_scale: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None):
    """Absorbed-MLA attention of q [B, T, H, 576] bf16 over the rows of
    kv [B, L, 576] (bf16, or uint8 e4m3 codes with kv_scale [B, L, 18]
    uint8 e8m0 or [B, L, 5] float32 tile scales) selected by idx [B, T, K]
    (-1 skipped).  Returns (out [B, T, H, 512] fp32, lse [B, T, H] fp32)."""
    B, T, H, D = q.shape
    L = kv.shape[1]
    K = idx.shape[2]
    _need(q, "q", torch.bfloat16, (B, T, H, LATENT))
    kd = _cache_dtype(kv, kv_scale, "kv", tiles_ok=True)
    _need(kv, "kv", kv.dtype, (B, L, LATENT))
    if kv_scale is not None:
        _need(kv_scale, "kv_scale", kv_scale.dtype,
              _scale_shape(kd, (B, L), LATENT))
    _need(idx, "idx", torch.int32, (B, T, K))
    dev = q.device
    if out is None:
        out = torch.empty((B, T, H, VALUE), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, (B, T, H, VALUE))
    _need(lse, "lse", torch.float32, (B, T, H))
    ws_bytes = workspace_size(OP_SPARSE_MLA, B, T, L, H, K)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    _check(_lib.dsa_sparse_mla_attn(
        B, T, L, H, K, _ptr(q), _ptr(kv), kd, _ptr(kv_scale), _ptr(idx),
        float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace),
        0 if workspace is None else workspace.numel(), _stream()),
        "dsa_sparse_mla_attn")
    return out, lse


@dataclass
class PagedCache:
    """One layer's paged cache: indexer keys and latent KV share one page
    table.  kidx [P, 64, d_I] and kv [P, 64, 576] are bf16, or uint8 e4m3
    codes with kidx_scale [P, 64, d_I/32] / kv_scale [P, 64, 18] uint8 e8m0;
    kv may also take float32 tile scales kv_scale [P, 64, 5].  page_table
    [B, max_pages] int32; seq_lens [B] int32."""
    kidx: torch.Tensor
    kv: torch.Tensor
    page_table: torch.Tensor
    seq_lens: torch.Tensor
    kidx_scale: Optional[torch.Tensor] = None
    kv_scale: Optional[torch.Tensor] = None

    def as_c(self) -> _PagedCacheC:
        P = self.kidx.shape[0]
        kd = _cache_dtype(self.kidx, self.kidx_scale, "kidx")
        vd = _cache_dtype(self.kv, self.kv_scale, "kv", tiles_ok=True)
        _need(self.kidx, "kidx", self.kidx.dtype)
        _need(self.kv, "kv", self.kv.dtype, (P, PAGE, LATENT))
        if self.kidx.dim() != 3 or self.kidx.shape[1] != PAGE:
            raise ValueError("kidx must be [num_pages, 64, d_I]")
        if self.kidx_scale is not None:
            _need(self.kidx_scale, "kidx_scale", torch.uint8,
                  (P, PAGE, self.kidx.shape[2] // 32))
        if self.kv_scale is not None:
            _need(self.kv_scale, "kv_scale", self.kv_scale.dtype,
                  _scale_shape(vd, (P, PAGE), LATENT))
        _need(self.page_table, "page_table", torch.int32)
        _need(self.seq_lens, "seq_lens", torch.int32,
              (self.page_table.shape[0],))
        return _PagedCacheC(PAGE, P, self.page_table.shape[1], kd, vd,
                            _ptr(self.kidx), _ptr(self.kidx_scale),
                            _ptr(self.kv), _ptr(self.kv_scale),
                            _ptr(self.page_table), _ptr(self.seq_lens))


def _decode_args(cache, q_idx, w, q, k, q_pos, out, lse, idx_out):
    """Shape checks and output allocation shared by the decode entry points."""
    B, T, H_I, d_I = q_idx.shape
    H = q.shape[2]
    _need(q_idx, "q_idx", torch.bfloat16)
    _need(w, "w", torch.float32, (B, T, H_I))
    _need(q, "q", torch.bfloat16, (B, T, H, LATENT))
    if q_pos is not None:
        _need(q_pos, "q_pos", torch.int32, (B, T))
    c = cache.as_c()
    if cache.kidx.shape[2] != d_I:
        raise ValueError(f"kidx rows are {cache.kidx.shape[2]} wide, the "
                         f"indexer queries {d_I}")
    if cache.page_table.shape[0] != B:
        raise ValueError(f"page_table has {cache.page_table.shape[0]} rows, "
                         f"the batch {B}")
    dev = q.device
    if out is None:
        out = torch.empty((B, T, H, VALUE), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, (B, T, H, VALUE))
    _need(lse, "lse", torch.float32, (B, T, H))
    if idx_out is not None:
        _need(idx_out, "idx_out", torch.int32, (B, T, k))
    return (B, T, H_I, d_I, H), c, out, lse


def decode_step(cache: PagedCache, q_idx: torch.Tensor, w: torch.Tensor,
                q: torch.Tensor, k: int, softmax_scale: float,
                max_seq_len: int, q_pos: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None,
                idx_out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None,
                quantize_queries: bool = False):
    """Indexer -> Top-K -> sparse attention for q_idx [B, T, H_I, d_I] bf16,
    w [B, T, H_I] fp32, q [B, T, H, 576] bf16 over a paged cache.  q_pos
    [B, T] int32, or None for T == 1 (the last cached token).
    quantize_queries as for indexer_scores.  Returns (out, lse, idx_out)."""
    (B, T, H_I, d_I, H), c, out, lse = _decode_args(
        cache, q_idx, w, q, k, q_pos, out, lse, idx_out)
    ws_bytes = workspace_size(OP_DECODE_STEP, B, T, max_seq_len, H, k)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8,
                                device=q.device)
    _check(_lib.dsa_decode_step(
        B, T, H_I, d_I, H, k, float(softmax_scale), ctypes.byref(c),
        int(max_seq_len), _ptr(q_idx),
        DSA_Q_MX32 if quantize_queries else DSA_Q_BF16, _ptr(w), _ptr(q),
        _ptr(q_pos),
        _ptr(out), _ptr(lse), _ptr(idx_out), _ptr(workspace),
        workspace.numel(), _stream()), "dsa_decode_step")
    return out, lse, idx_out


def decode_step_static(cache: PagedCache, q_idx: torch.Tensor,
                       w: torch.Tensor, q: torch.Tensor, k: int,
                       softmax_scale: float, max_seq_len: int,
                       q_pos: Optional[torch.Tensor] = None,
                       out: Optional[torch.Tensor] = None,
                       lse: Optional[torch.Tensor] = None,
                       idx_out: Optional[torch.Tensor] = None,
                       quantize_queries: bool = False):
    """decode_step without a workspace: the library's static device scratch
    (STATIC_SCRATCH_BYTES per GPU) holds the intermediates, and the library
    call allocates nothing (pass out / lse to allocate nothing here either).
    Calls that overlap on one GPU share that scratch and race."""
    (B, T, H_I, d_I, H), c, out, lse = _decode_args(
        cache, q_idx, w, q, k, q_pos, out, lse, idx_out)
    _check(_lib.dsa_decode_step_static(
        B, T, H_I, d_I, H, k, float(softmax_scale), ctypes.byref(c),
        int(max_seq_len), _ptr(q_idx),
        DSA_Q_MX32 if quantize_queries else DSA_Q_BF16, _ptr(w), _ptr(q),
        _ptr(q_pos), _ptr(out), _ptr(lse), _ptr(idx_out), _stream()),
        "dsa_decode_step_static")
    return out, lse, idx_out


def indexer_topk(cache: PagedCache, q_idx: torch.Tensor, w: torch.Tensor,
                 k: int, max_seq_len: int,
                 q_pos: Optional[torch.Tensor] = None,
                 idx_out: Optional[torch.Tensor] = None,
                 quantize_queries: bool = False):
    """Indexer scores and Top-K of every query row in one kernel (the scores
    never leave the chip) for q_idx [B, T, H_I, d_I] bf16 and w [B, T, H_I]
    fp32 over the paged key cache; max_seq_len <= FUSED_MAX_CONTEXT.  q_pos
    [B, T] int32, or None for T == 1.  quantize_queries as for
    indexer_scores (MX keys).  Returns idx [B, T, k] int32, the same
    selection as indexer_scores followed by topk."""
    B, T, H_I, d_I = q_idx.shape
    _need(q_idx, "q_idx", torch.bfloat16)
    _need(w, "w", torch.float32, (B, T, H_I))
    if q_pos is not None:
        _need(q_pos, "q_pos", torch.int32, (B, T))
    c = cache.as_c()
    if cache.kidx.shape[2] != d_I:
        raise ValueError(f"kidx rows are {cache.kidx.shape[2]} wide, the "
                         f"indexer queries {d_I}")
    if cache.page_table.shape[0] != B:
        raise ValueError(f"page_table has {cache.page_table.shape[0]} rows, "
                         f"the batch {B}")
    if idx_out is None:
        idx_out = torch.empty((B, T, k), dtype=torch.int32,
                              device=q_idx.device)
    _need(idx_out, "idx_out", torch.int32, (B, T, k))
    _check(_lib.dsa_indexer_topk(
        B, T, H_I, d_I, k, ctypes.byref(c), int(max_seq_len), _ptr(q_idx),
        DSA_Q_MX32 if quantize_queries else DSA_Q_BF16, _ptr(w), _ptr(q_pos),
        _ptr(idx_out), _stream()),
        "dsa_indexer_topk")
    return idx_out


def cache_append(cache: PagedCache, pos: torch.Tensor,
                 k_new: Optional[torch.Tensor] = None,
                 kv_new: Optional[torch.Tensor] = None) -> None:
    """Store new tokens into ``cache``'s pools, in place: k_new [B, T, d_I]
    and / or kv_new [B, T, 576] bf16 rows go to the slots of the logical
    positions pos [B, T] int32 (pos < 0 skipped), quantised to the pools'
    formats.  seq_lens is left to the caller."""
    if k_new is None and kv_new is None:
        raise ValueError("cache_append: nothing to append")
    c = cache.as_c()
    _need(pos, "pos", torch.int32)
    if pos.dim() != 2:
        raise ValueError("pos must be [B, T]")
    B, T = pos.shape
    if cache.page_table.shape[0] != B:
        raise ValueError("pos and page_table disagree on B")
    d_I = cache.kidx.shape[2]
    if k_new is not None:
        _need(k_new, "k_new", torch.bfloat16, (B, T, d_I))
    if kv_new is not None:
        _need(kv_new, "kv_new", torch.bfloat16, (B, T, LATENT))
    _check(_lib.dsa_cache_append(
        B, T, d_I, c.num_pages, c.max_pages_per_seq, _ptr(cache.page_table),
        _ptr(pos), _ptr(k_new), c.kidx_dtype, _ptr(cache.kidx),
        _ptr(cache.kidx_scale), _ptr(kv_new), c.kv_dtype, _ptr(cache.kv),
        _ptr(cache.kv_scale), _stream()), "dsa_cache_append")


def default_softmax_scale() -> float:
    """1/sqrt(192): the un-absorbed MLA query-key width (128 + 64)."""
    return 1.0 / math.sqrt(192.0)
