"""The C-ABI library on the host (no GPU needed): it loads, exports every
entry point include/dsa.h declares, and rejects bad arguments with the
documented status codes before any HIP call."""
import ctypes
import os
import re

import pytest

import indexed_sparse_attention_lightning_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")
lib = dsa._lib

OK, NULL, SHAPE, UNSUP, WS = 0, 1, 2, 3, 4
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:dsa_status|size_t|const char\*)\s+"
                                 r"(dsa_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("dsa_indexer_scores", "dsa_topk", "dsa_sparse_mla_attn",
              "dsa_decode_step", "dsa_cache_append", "dsa_workspace_size",
              "dsa_status_string", "dsa_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    so = ctypes.CDLL(dsa.library_path())
    for n in declared_functions():
        assert hasattr(so, n), n


def test_status_strings():
    for code in range(6):
        assert lib.dsa_status_string(code).decode().startswith("DSA_")
    assert b"unknown" in lib.dsa_status_string(99)


def scores_call(**kw):
    a = dict(B=1, T=1, L=64, H_I=64, d_I=128, q=FAKE, qm=0, w=FAKE, k=FAKE,
             kd=0, ks=None, qp=FAKE, out=FAKE)
    a.update(kw)
    return lib.dsa_indexer_scores(a["B"], a["T"], a["L"], a["H_I"], a["d_I"],
                                  a["q"], a["qm"], a["w"], a["k"], a["kd"],
                                  a["ks"], a["qp"], a["out"], None)


def test_indexer_scores_validation():
    assert scores_call(q=None) == NULL
    assert scores_call(out=None) == NULL
    assert scores_call(B=0) == SHAPE
    assert scores_call(L=0) == SHAPE
    assert scores_call(H_I=65) == UNSUP
    assert scores_call(d_I=96) == UNSUP
    assert scores_call(kd=7) == UNSUP
    assert scores_call(kd=1, ks=None) == NULL
    assert scores_call(qm=2) == UNSUP             # unknown query mode
    assert scores_call(qm=1) == UNSUP             # quantised queries: MX keys
    assert scores_call(qm=1, kd=1, ks=FAKE, q=None) == NULL
    assert b"d_I" in lib.dsa_last_error() or True


def test_topk_validation():
    f = lambda **kw: lib.dsa_topk(kw.get("B", 1), 1, kw.get("L", 64),
                                  kw.get("K", 8), kw.get("s", FAKE), FAKE,
                                  kw.get("i", FAKE), None, 0, None)
    assert f(s=None) == NULL
    assert f(i=None) == NULL
    assert f(L=0) == SHAPE
    assert f(K=0) == UNSUP
    assert f(K=4097) == UNSUP
    assert f(L=131073) == UNSUP


def test_sparse_mla_validation():
    def f(**kw):
        a = dict(B=1, T=1, L=64, H=128, K=64, kd=0, ks=None, ws=None, wsb=0)
        a.update(kw)
        return lib.dsa_sparse_mla_attn(a["B"], a["T"], a["L"], a["H"], a["K"],
                                       FAKE, FAKE, a["kd"], a["ks"], FAKE,
                                       a.get("scale", 0.1),
                                       FAKE, FAKE, a["ws"], a["wsb"], None)
    assert f(scale=0.0) == SHAPE                # the softmax scale must be > 0
    assert f(scale=-0.1) == SHAPE
    assert f(scale=float("inf")) == SHAPE
    assert f(scale=float("nan")) == SHAPE
    assert f(H=129) == UNSUP
    assert f(K=0) == UNSUP
    assert f(kd=1) == NULL
    assert f(kd=2) == NULL                      # tile scales too
    assert f(kd=3) == UNSUP
    # 32 tokens split their rows: a workspace is needed
    assert f(B=32, K=2048) == WS
    need = dsa.workspace_size(dsa.OP_SPARSE_MLA, 32, 1, 64, 128, 2048)
    assert need > 0
    assert f(B=32, K=2048, ws=FAKE, wsb=need - 1) == WS


def test_decode_step_validation():
    c = dsa._PagedCacheC(64, 10, 4, 0, 0, 0x1000, None, 0x1000, None, 0x1000,
                         0x1000)

    def f(cache=c, **kw):
        a = dict(B=2, T=1, H_I=64, d_I=128, H=128, K=64, msl=256, qp=None,
                 ws=FAKE, wsb=1 << 40, qm=0)
        a.update(kw)
        return lib.dsa_decode_step(a["B"], a["T"], a["H_I"], a["d_I"], a["H"],
                                   a["K"], 0.07, ctypes.byref(cache) if cache
                                   else None, a["msl"], FAKE, a["qm"], FAKE,
                                   FAKE, a["qp"], FAKE, FAKE, None, a["ws"],
                                   a["wsb"], None)
    assert f(cache=None) == NULL
    assert f(qm=1) == UNSUP                     # quantised queries: MX keys
    assert f(qm=-1) == UNSUP
    assert f(T=2) == NULL                       # q_pos required for T > 1
    assert f(msl=257) == SHAPE                  # beyond max_pages * 64
    assert f(ws=None) == WS
    need = dsa.workspace_size(dsa.OP_DECODE_STEP, 2, 1, 256, 128, 64)
    assert f(wsb=need - 1) == WS
    bad = dsa._PagedCacheC(32, 10, 4, 0, 0, 0x1000, None, 0x1000, None,
                           0x1000, 0x1000)
    assert f(cache=bad) == UNSUP                # page size must be 64
    fp8 = dsa._PagedCacheC(64, 10, 4, 1, 0, 0x1000, None, 0x1000, None,
                           0x1000, 0x1000)
    assert f(cache=fp8) == NULL                 # MX keys need scales
    t128_keys = dsa._PagedCacheC(64, 10, 4, 2, 0, 0x1000, 0x1000, 0x1000,
                                 None, 0x1000, 0x1000)
    assert f(cache=t128_keys) == UNSUP          # tiles are for the KV only
    t128_kv = dsa._PagedCacheC(64, 10, 4, 0, 2, 0x1000, None, 0x1000, None,
                               0x1000, 0x1000)
    assert f(cache=t128_kv) == NULL             # tile scales missing


def test_cache_append_validation():
    def f(**kw):
        a = dict(B=2, T=1, d_I=128, P=10, MP=4, pt=FAKE, pos=FAKE, kn=FAKE,
                 kd=0, k=FAKE, ks=None, vn=FAKE, vd=0, v=FAKE, vs=None)
        a.update(kw)
        return lib.dsa_cache_append(a["B"], a["T"], a["d_I"], a["P"], a["MP"],
                                    a["pt"], a["pos"], a["kn"], a["kd"],
                                    a["k"], a["ks"], a["vn"], a["vd"], a["v"],
                                    a["vs"], None)
    assert f(pt=None) == NULL
    assert f(pos=None) == NULL
    assert f(kn=None, vn=None) == NULL          # nothing to append
    assert f(B=0) == SHAPE
    assert f(T=0) == SHAPE
    assert f(P=0) == SHAPE
    assert f(MP=0) == SHAPE
    assert f(d_I=96) == UNSUP
    assert f(kd=2) == UNSUP                     # keys: bf16 or MX32 only
    assert f(kd=1) == NULL                      # MX keys need their scales
    assert f(k=None) == NULL
    assert f(vd=5) == UNSUP
    assert f(vd=1) == NULL
    assert f(vd=2) == NULL
    assert f(v=None) == NULL
    # a pool that is not appended to is not checked
    assert f(kn=None, d_I=96, kd=9, k=None, vd=7, vn=None) == NULL
    assert b"dsa_cache_append" in lib.dsa_last_error() or \
        b"neither" in lib.dsa_last_error()


def test_workspace_sizes():
    assert dsa.workspace_size(dsa.OP_TOPK, 32, 1, 32768, 128, 2048) == 0
    d = dsa.workspace_size(dsa.OP_DECODE_STEP, 32, 1, 32768, 128, 2048)
    # scores + indices at least
    assert d >= 32 * 32768 * 4 + 32 * 2048 * 4
    assert dsa.workspace_size(99, 1, 1, 1, 1, 1) == 0


def test_decode_step_static_validation():
    """The static-scratch decode step validates like dsa_decode_step and
    refuses sizes whose workspace exceeds its scratch before any HIP call."""
    c = dsa._PagedCacheC(64, 10, 2048, 0, 0, 0x1000, None, 0x1000, None,
                         0x1000, 0x1000)

    def f(cache=c, **kw):
        a = dict(B=2, T=1, H_I=64, d_I=128, H=128, K=64, msl=256, qp=None)
        a.update(kw)
        return lib.dsa_decode_step_static(
            a["B"], a["T"], a["H_I"], a["d_I"], a["H"], a["K"], 0.07,
            ctypes.byref(cache) if cache else None, a["msl"], FAKE, 0, FAKE,
            FAKE, a["qp"], FAKE, FAKE, None, None)
    assert f(cache=None) == NULL
    assert f(H=129) == UNSUP
    big = dict(B=200, msl=131072)
    assert dsa.workspace_size(dsa.OP_DECODE_STEP, 200, 1, 131072, 128,
                              64) > dsa.STATIC_SCRATCH_BYTES
    assert f(**big) == WS
    assert b"static scratch" in lib.dsa_last_error()


def test_indexer_topk_validation():
    """The fused indexer + Top-K checks its arguments before any HIP call:
    rows beyond the LDS bound, quantised queries without MX keys and the
    cache fields it reads."""
    c = dsa._PagedCacheC(64, 10, 1024, 0, 0, 0x1000, None, None, None,
                         0x1000, 0x1000)

    def f(cache=c, **kw):
        a = dict(B=2, T=1, H_I=64, d_I=128, K=64, msl=256, qp=None, qm=0,
                 out=FAKE)
        a.update(kw)
        return lib.dsa_indexer_topk(a["B"], a["T"], a["H_I"], a["d_I"], a["K"],
                                    ctypes.byref(cache) if cache else None,
                                    a["msl"], FAKE, a["qm"], FAKE, a["qp"],
                                    a["out"], None)
    assert f(cache=None) == NULL
    assert f(out=None) == NULL
    assert f(T=2) == NULL                       # q_pos required for T > 1
    assert f(K=0) == UNSUP and f(K=2049) == UNSUP
    assert f(H_I=65) == UNSUP and f(d_I=96) == UNSUP
    assert f(msl=dsa.FUSED_MAX_CONTEXT + 1) == UNSUP
    assert b"LDS" in lib.dsa_last_error()
    assert f(msl=0) == SHAPE
    short = dsa._PagedCacheC(64, 10, 4, 0, 0, 0x1000, None, None, None,
                             0x1000, 0x1000)
    assert f(cache=short, msl=257) == SHAPE     # beyond max_pages * 64
    assert f(qm=-1) == UNSUP
    assert f(qm=1) == UNSUP                     # quantised queries: MX keys
    assert b"MX32 keys" in lib.dsa_last_error()
    assert f(cache=dsa._PagedCacheC(64, 10, 1024, 1, 0, 0x1000, None, None,
                                    None, 0x1000, 0x1000)) == NULL
    assert f(cache=dsa._PagedCacheC(64, 10, 1024, 2, 0, 0x1000, 0x1000, None,
                                    None, 0x1000, 0x1000)) == UNSUP
    assert f(cache=dsa._PagedCacheC(64, 10, 1024, 0, 0, 0x1000, None, None,
                                    None, None, 0x1000)) == NULL
