"""Seeded synthetic inputs for the indexed sparse attention (DSA) hot path.

This module is shared by the CPU oracle and by the HIP path's tests and
benchmark.  It draws random numbers and lays them out in the storage formats
the C-ABI receives (bf16 bit patterns, e4m3fn codes with e8m0 block scales,
page tables).  It holds none of the method's arithmetic: no scoring, no
selection, no attention.  The MX block quantiser below is the *input* side of
the quantized configurations (the caches arrive already quantized); the hot
path itself only ever decodes.

Workloads (one DSA layer, synthetic, no trained weights):

* ``tiny``      batch 1, one query at position 511 over L=512; H_I=4, d_I=64;
                top_k=64; 16 MLA heads; integer keys/queries in [-3, 3].
* ``decode``    batch 32, every sequence at L=32768, contiguous cache;
                H_I=64, d_I=128, top_k=2048, 128 MLA heads; integers in [-4, 4].
* ``decode_fp8`` the ``decode`` tensors, with indexer keys as e4m3 and the
                latent KV as MXFP8 (block 32 along features, e8m0 scales).
* ``prefill``   4096 queries at positions 61440..65535 of a 65536-token
                context, bf16.
* ``ragged``    batch 4, lengths uniform in [16384, 131072], 64-token pages
                scattered by a seeded page table, FP8 keys and MXFP8 KV.

Draw order for a workload with seed ``s`` (``numpy.random.default_rng(s)``):
(ragged only: lengths [B], then the page permutation), indexer queries
(integers), indexer keys (integers), the head-weight exponents ``u``, MLA
queries (N(0,1)), latent KV (N(0,1)).  ``decode_fp8`` reuses the draws of
``decode`` (same seed) and quantizes them.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

D_LATENT = 576      # absorbed MLA key width: 512 latent ("nope") + 64 rope
D_VALUE = 512       # value width: the first 512 latent features
MX_BLOCK = 32       # MX block size along the feature dimension
PAGE_SIZE = 64      # tokens per cache page
E4M3_MAX = 448.0    # largest finite e4m3fn magnitude

# bit patterns used to poison cache slots that lie beyond a sequence's length
BF16_NAN_BITS = 0x7FC0
E4M3_NAN_CODE = 0x7F
E8M0_NAN_CODE = 0xFF


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    T: int
    H_I: int
    d_I: int
    top_k: int
    H: int
    int_range: int            # indexer q/k are integers uniform in [-r, r]
    quantized: bool           # e4m3+e8m0 indexer keys and MXFP8 latent KV
    paged_random: bool        # pages scattered by a seeded permutation
    L: Optional[int] = None   # fixed context length (None: drawn per sequence)
    L_min: int = 0
    L_max: int = 0
    first_pos: Optional[int] = None   # position of the first query (T > 1)
    softmax_scale: float = 1.0 / np.sqrt(192.0)


WORKLOADS = {
    "tiny": Workload("tiny", 0, B=1, T=1, H_I=4, d_I=64, top_k=64, H=16,
                     int_range=3, quantized=False, paged_random=False, L=512),
    "decode": Workload("decode", 1, B=32, T=1, H_I=64, d_I=128, top_k=2048,
                       H=128, int_range=4, quantized=False,
                       paged_random=False, L=32768),
    "decode_fp8": Workload("decode_fp8", 1, B=32, T=1, H_I=64, d_I=128,
                           top_k=2048, H=128, int_range=4, quantized=True,
                           paged_random=False, L=32768),
    "prefill": Workload("prefill", 3, B=1, T=4096, H_I=64, d_I=128,
                        top_k=2048, H=128, int_range=4, quantized=False,
                        paged_random=False, L=65536, first_pos=61440),
    "ragged": Workload("ragged", 4, B=4, T=1, H_I=64, d_I=128, top_k=2048,
                       H=128, int_range=4, quantized=True, paged_random=True,
                       L_min=16384, L_max=131072),
}


def scaled(wl: Workload, **changes) -> Workload:
    """A smaller (or otherwise modified) copy of a workload, for tests."""
    return dataclasses.replace(wl, **changes)


# ---------------------------------------------------------------- encodings

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bf16, returned as uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def mx32_quantize(x: np.ndarray):
    """MX block-32 quantisation of the last axis (input generation only).

    Each block of 32 features gets one power-of-two scale 2^X with X the
    smallest integer such that 448 * 2^X >= amax(block), so no element
    saturates; elements are rounded to nearest-even e4m3fn.  An all-zero block
    gets X = 0.  Returns (codes uint8 [..., n], scale codes uint8 [..., n/32])
    where a scale code is X + 127 (e8m0).
    """
    x = np.asarray(x, dtype=np.float32)
    n = x.shape[-1]
    assert n % MX_BLOCK == 0
    blocks = x.reshape(*x.shape[:-1], n // MX_BLOCK, MX_BLOCK)
    amax = np.abs(blocks).max(axis=-1).astype(np.float64)
    _, e = np.frexp(np.where(amax > 0, amax / E4M3_MAX, 1.0))
    X = e.astype(np.int64)               # 2^(e-1) <= amax/448 < 2^e
    # settle X exactly: smallest X with 448*2^X >= amax (all steps exact)
    for _ in range(2):
        X = np.where(np.ldexp(E4M3_MAX, X - 1) >= amax, X - 1, X)
    X = np.where(np.ldexp(E4M3_MAX, X) < amax, X + 1, X)
    X = np.where(amax > 0, X, 0)
    assert X.min() >= -127 and X.max() <= 127
    scaled_blocks = blocks.astype(np.float64) / np.ldexp(1.0, X)[..., None]
    t = torch.from_numpy(scaled_blocks.astype(np.float32))
    codes = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return (codes.reshape(x.shape).copy(),
            (X + 127).astype(np.uint8))


def append_rows(seed: int, n: int, width: int) -> np.ndarray:
    """bf16 bit patterns [n, width] of new cache rows, drawn to exercise the
    cache-append quantizers: row kind i % 8 is
      0 normal values times a per-row magnitude over a wide exponent range
      1 normal values with some 32-groups zeroed and some -0.0 entries
      2 tiny magnitudes, down into the bf16 subnormals
      3 very large magnitudes, up to near the bf16 maximum
      4 per 32-group: one element of magnitude 448 * 2^k, the rest exact
        midpoints between neighbouring 3-bit-mantissa values times 2^k
      5 small integers in [-4, 4]
      6 one non-zero element per 32-group
      7 uniform values with a different power-of-two magnitude per group
    """
    assert width % 32 == 0
    rng = np.random.default_rng(seed)
    g = width // 32
    out = np.empty((n, width), dtype=np.float32)
    for i in range(n):
        kind = i % 8
        if kind == 0:
            r = rng.standard_normal(width) * np.exp(3 * rng.standard_normal())
        elif kind == 1:
            r = rng.standard_normal(width)
            r.reshape(g, 32)[rng.random(g) < 0.4] = 0.0
            r[rng.random(width) < 0.05] = -0.0
        elif kind == 2:
            r = rng.standard_normal(width) * np.ldexp(1.0, rng.integers(-136, -120))
        elif kind == 3:
            r = rng.uniform(-1, 1, width) * np.ldexp(1.0, rng.integers(100, 127))
        elif kind == 4:
            k = rng.integers(-20, 20, size=g)
            m = rng.integers(0, 7, size=(g, 32))
            e = rng.integers(-5, 8, size=(g, 32))
            mid = (1.0 + (2 * m + 1) / 16.0) * np.ldexp(1.0, e)
            mid *= rng.choice([-1.0, 1.0], size=(g, 32))
            mid[np.arange(g), rng.integers(0, 32, size=g)] = \
                E4M3_MAX * rng.choice([-1.0, 1.0], size=g)
            r = (mid * np.ldexp(1.0, k)[:, None]).reshape(width)
        elif kind == 5:
            r = rng.integers(-4, 5, size=width).astype(np.float64)
        elif kind == 6:
            r = np.zeros((g, 32))
            r[np.arange(g), rng.integers(0, 32, size=g)] = \
                rng.standard_normal(g) * 10.0
            r = r.reshape(width)
        else:
            r = (rng.uniform(-1, 1, (g, 32)) *
                 np.ldexp(1.0, rng.integers(-30, 30, size=g))[:, None])
            r = r.reshape(width)
        out[i] = r
    return f32_to_bf16_bits(out)


def eighths(seed: int, shape, limit: int = 39) -> np.ndarray:
    """bf16 bit patterns of k/8 for integers k uniform in [-limit, limit]:
    indexer queries with fractional parts (inputs of the quantised-indexer
    tests; multiples of 1/8 keep every indexer sum exact in fp32)."""
    rng = np.random.default_rng(seed)
    k = rng.integers(-limit, limit + 1, size=shape)
    return f32_to_bf16_bits((k / 8.0).astype(np.float32))


# ---------------------------------------------------------------- caches

@dataclasses.dataclass
class Cache:
    """One layer's cache in the storage the C-ABI receives.

    Rows live in pages of ``page_size`` tokens: ``data`` is
    [num_pages, page_size, width] (uint16 bf16 bits, or uint8 e4m3 codes) and
    ``scale`` is [num_pages, page_size, width/32] e8m0 codes (quantized only).
    A contiguous [B, L, width] cache is the same storage with an identity page
    table (sequence b owns pages b*L/64 .. (b+1)*L/64 - 1).
    """
    data: np.ndarray
    scale: Optional[np.ndarray]
    quantized: bool

    @property
    def width(self) -> int:
        return self.data.shape[-1]


@dataclasses.dataclass
class Inputs:
    wl: Workload
    seq_lens: np.ndarray      # int32 [B], tokens in cache incl. current ones
    q_pos: np.ndarray         # int32 [B, T]
    page_table: np.ndarray    # int32 [B, max_pages], -1 where unused
    q_idx: np.ndarray         # uint16 bf16 bits [B, T, H_I, d_I]
    w: np.ndarray             # float32 [B, T, H_I]
    q: np.ndarray             # uint16 bf16 bits [B, T, H, 576]
    k_idx: Cache              # indexer keys, width d_I
    kv: Cache                 # latent KV, width 576
    contiguous: bool          # identity page table with fixed L

    @property
    def L(self) -> int:
        """Context length of the contiguous layout (max length if ragged)."""
        return int(self.seq_lens.max())

    def contiguous_view(self, cache: Cache):
        """[B, L, width] views of a contiguous cache (data, scale-or-None)."""
        assert self.contiguous
        B, L = self.wl.B, self.L
        d = cache.data.reshape(B, L, cache.width)
        s = None if cache.scale is None else cache.scale.reshape(B, L, -1)
        return d, s


def _int_draw(rng, r, shape):
    return rng.integers(-r, r + 1, size=shape, dtype=np.int64).astype(np.float32)


def _normal_draw(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def _place_pages(rows: np.ndarray, starts, lens, page_of, num_pages, fill):
    """Scatter per-sequence row blocks into 64-token pages.

    ``rows`` is [sum(lens), width]; sequence b's rows start at starts[b].
    Slots past a sequence's length (the tail of its last page) hold ``fill``.
    """
    width = rows.shape[-1]
    out = np.full((num_pages, PAGE_SIZE, width), fill, dtype=rows.dtype)
    for b, (st, n) in enumerate(zip(starts, lens)):
        npg = -(-n // PAGE_SIZE)
        pad = npg * PAGE_SIZE - n
        blk = rows[st:st + n]
        if pad:
            blk = np.concatenate(
                [blk, np.full((pad, width), fill, dtype=rows.dtype)])
        out[page_of[b][:npg]] = blk.reshape(npg, PAGE_SIZE, width)
    return out


def generate(wl: Workload) -> Inputs:
    """Draw one workload's inputs (deterministic in ``wl.seed``)."""
    rng = np.random.default_rng(wl.seed)
    B, T = wl.B, wl.T
    if wl.L is not None:
        lens = np.full(B, wl.L, dtype=np.int64)
    else:
        lens = rng.integers(wl.L_min, wl.L_max + 1, size=B, dtype=np.int64)
    npages = -(-lens // PAGE_SIZE)
    num_pages = int(npages.sum())
    max_pages = int(npages.max())
    if wl.paged_random:
        perm = rng.permutation(num_pages)
    else:
        perm = np.arange(num_pages)
    page_of, off = [], 0
    page_table = np.full((B, max_pages), -1, dtype=np.int32)
    for b in range(B):
        pg = perm[off:off + npages[b]]
        page_of.append(pg)
        page_table[b, :npages[b]] = pg
        off += npages[b]

    if T == 1:
        q_pos = (lens - 1).reshape(B, 1)
    else:
        assert wl.first_pos is not None
        q_pos = np.broadcast_to(wl.first_pos + np.arange(T), (B, T))
        assert q_pos.max() < lens.min()
    q_pos = np.ascontiguousarray(q_pos, dtype=np.int32)

    total = int(lens.sum())
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    qi = _int_draw(rng, wl.int_range, (B, T, wl.H_I, wl.d_I))
    ki = _int_draw(rng, wl.int_range, (total, wl.d_I))
    u = rng.integers(0, 4, size=(B, T, wl.H_I), dtype=np.int64)
    w = np.ldexp(np.float32(1.0), -u).astype(np.float32)
    q = _normal_draw(rng, (B, T, wl.H, D_LATENT))
    kv = _normal_draw(rng, (total, D_LATENT))

    if wl.quantized:
        kc, ks = mx32_quantize(ki)
        vc, vs = mx32_quantize(kv)
        del kv
        k_cache = Cache(
            _place_pages(kc, starts, lens, page_of, num_pages, E4M3_NAN_CODE),
            _place_pages(ks, starts, lens, page_of, num_pages, E8M0_NAN_CODE),
            True)
        kv_cache = Cache(
            _place_pages(vc, starts, lens, page_of, num_pages, E4M3_NAN_CODE),
            _place_pages(vs, starts, lens, page_of, num_pages, E8M0_NAN_CODE),
            True)
    else:
        k_cache = Cache(_place_pages(f32_to_bf16_bits(ki), starts, lens,
                                     page_of, num_pages, BF16_NAN_BITS),
                        None, False)
        kvb = f32_to_bf16_bits(kv)
        del kv
        kv_cache = Cache(_place_pages(kvb, starts, lens, page_of, num_pages,
                                      BF16_NAN_BITS), None, False)

    contiguous = (not wl.paged_random) and wl.L is not None \
        and wl.L % PAGE_SIZE == 0
    return Inputs(wl=wl, seq_lens=lens.astype(np.int32), q_pos=q_pos,
                  page_table=page_table, q_idx=f32_to_bf16_bits(qi), w=w,
                  q=f32_to_bf16_bits(q), k_idx=k_cache, kv=kv_cache,
                  contiguous=contiguous)
