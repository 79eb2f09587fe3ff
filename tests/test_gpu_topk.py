"""dsa_topk on score rows of every shape class vs the oracle's Top-K.

Rows cover each workgroup shape of the kernel (rows up to 4K, 16K, 32K and
64K positions keep their keys in registers; longer rows re-read them) and
score distributions that stress the digit passes: heavy ties, a few
distinct values, NaN / +-inf / -0 / subnormals, huge dynamic range, and
the indexer's own distribution (multiples of 1/8 in a narrow band); and
rows far from normal: light and heavy tails, two clusters, all-negative
rows, far outliers, and a spike row with K - 1 keys above a constant.
Index sets must match exactly.
"""
import numpy as np
import pytest
import torch

import indexed_sparse_attention_lightning_amd as dsa
import oracle

pytestmark = pytest.mark.gpu


def _rows(kind, rng, R, L, K=2048):
    if kind == "normal":
        return rng.standard_normal((R, L)).astype(np.float32)
    if kind == "indexer_like":
        return (200.0 + rng.integers(0, 14400, (R, L)) / 8.0).astype(np.float32)
    if kind == "few_values":
        return rng.integers(-2, 3, (R, L)).astype(np.float32)
    if kind == "specials":
        x = (rng.standard_normal((R, L)) * 1e30).astype(np.float32)
        vals = np.array([np.nan, np.inf, -np.inf, -0.0, 0.0, 1e-45, -1e-45],
                        dtype=np.float32)
        m = rng.random((R, L)) < 0.3
        x[m] = rng.choice(vals, size=int(m.sum()))
        return x
    if kind == "all_equal":
        return np.full((R, L), 7.5, dtype=np.float32)
    if kind == "uniform":
        return rng.random((R, L)).astype(np.float32)
    if kind == "heavy_tail":
        return (rng.standard_exponential((R, L)) ** 3).astype(np.float32)
    if kind == "two_clusters":
        x = rng.standard_normal((R, L))
        x[rng.random((R, L)) < 0.1] += 50.0
        return x.astype(np.float32)
    if kind == "negative":
        return (-1000.0 + rng.standard_normal((R, L))).astype(np.float32)
    if kind == "outlier":
        x = rng.standard_normal((R, L)).astype(np.float32)
        x[:, ::977] = 3e37
        return x
    if kind == "spike":
        x = np.ones((R, L), dtype=np.float32)
        for r in range(R):
            x[r, rng.choice(L, size=min(K - 1, L), replace=False)] = 2.0
        return x
    raise ValueError(kind)


KINDS = ["normal", "indexer_like", "few_values", "specials", "all_equal",
         "uniform", "heavy_tail", "two_clusters", "negative", "outlier",
         "spike"]
LENGTHS = [700, 4096, 9000, 32768, 50000, 65536, 100000, 131072]


@pytest.mark.parametrize("L", LENGTHS)
def test_topk_lengths_and_distributions(L):
    rng = np.random.default_rng(1000 + L)
    K = 2048 if L > 4096 else 300
    for kind in KINDS:
        R = 3
        x = _rows(kind, rng, R, L, K)
        # causal extents: full row, a ragged middle, and one short of K
        q_pos = np.array([[L - 1], [int(rng.integers(K, L))],
                          [min(K - 2, L - 1)]], dtype=np.int32)
        scores = torch.from_numpy(x).view(R, 1, L).cuda()
        idx = dsa.topk(scores, torch.from_numpy(q_pos).cuda(), K)
        torch.cuda.synchronize()
        got = idx.cpu().numpy()
        for r in range(R):
            want = oracle.topk_row(x[r], int(q_pos[r, 0]), K)
            assert np.array_equal(got[r, 0], want), \
                f"{kind} L={L} row {r} q_pos={q_pos[r, 0]}"


@pytest.mark.parametrize("L", [65537, 100000, 131072])
def test_topk_long_rows_one_workgroup_path(L):
    """Rows past 64K positions without a workspace: one workgroup streams the
    whole row (the chunk-candidate path is covered above)."""
    rng = np.random.default_rng(2000 + L)
    K = 2048
    for kind in ("indexer_like", "few_values", "specials"):
        x = _rows(kind, rng, 2, L)
        q_pos = np.array([[L - 1], [int(rng.integers(K, L))]], dtype=np.int32)
        scores = torch.from_numpy(x).view(2, 1, L).cuda()
        idx = dsa.topk(scores, torch.from_numpy(q_pos).cuda(), K,
                       workspace=torch.empty(0, dtype=torch.uint8,
                                             device="cuda"))
        torch.cuda.synchronize()
        got = idx.cpu().numpy()
        for r in range(2):
            want = oracle.topk_row(x[r], int(q_pos[r, 0]), K)
            assert np.array_equal(got[r, 0], want), f"{kind} L={L} row {r}"


def test_topk_long_rows_chunk_boundaries():
    """Candidate lists of 16K-position chunks: equal scores straddling chunk
    boundaries, selections concentrated in one chunk, causal extents ending
    inside a chunk, and K = 1."""
    rng = np.random.default_rng(31)
    L = 70000
    x = np.zeros((4, L), dtype=np.float32)
    x[0] = 1.0
    x[0, 16384 - 1000:16384 + 1000] = 2.0        # 2000 equal keys across a boundary
    x[1] = rng.standard_normal(L).astype(np.float32)
    x[1, 49152:49152 + 3000] += 100.0           # the whole Top-K in one chunk
    x[2] = rng.integers(0, 3, L).astype(np.float32)
    x[3] = rng.standard_normal(L).astype(np.float32)
    q_pos = np.array([[L - 1], [L - 1], [40000], [16383 + 5]], dtype=np.int32)
    scores = torch.from_numpy(x).view(4, 1, L).cuda()
    qp = torch.from_numpy(q_pos).cuda()
    for K in (2048, 1, 777):
        idx = dsa.topk(scores, qp, K)
        torch.cuda.synchronize()
        got = idx.cpu().numpy()
        for r in range(4):
            want = oracle.topk_row(x[r], int(q_pos[r, 0]), K)
            assert np.array_equal(got[r, 0], want), f"K={K} row {r}"


def test_topk_many_rows_prefill_shape():
    """Many rows with staggered causal extents in one launch (the prefill
    chunk's row structure), unaligned row length."""
    rng = np.random.default_rng(77)
    T, L, K = 64, 20001, 512
    x = (rng.integers(-40, 41, (T, L)) / 4.0).astype(np.float32)
    q_pos = (L - T + np.arange(T, dtype=np.int32)).reshape(1, T)
    q_pos[0, :8] = np.array([0, 1, 5, 510, 511, 512, 513, 9999])
    scores = torch.from_numpy(x).view(1, T, L).cuda()
    idx = dsa.topk(scores, torch.from_numpy(q_pos).cuda(), K)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for t in range(T):
        want = oracle.topk_row(x[t], int(q_pos[0, t]), K)
        assert np.array_equal(got[0, t], want), f"row {t}"


@pytest.mark.parametrize("L", [4096, 32768, 65536, 100000])
def test_topk_threshold_digit_sizes(L):
    """Rows whose threshold digit (after the first digit pass) holds 63, 64
    or 65 keys -- at most 64 take the one-wave finish, more the remaining
    digit passes -- with equal keys in it that the K-th position splits: both
    finishes must take the higher keys, then the lower positions.  K - 40
    keys lie far above (1000 + i), a cluster of eight distinct values in
    [50, 50.11] (one first-pass digit: the row's key range spans about 2^28,
    so a digit covers 2^18 or 2^19 float steps, at least 1.0 at 50) holds the
    threshold, the rest lie in [0, 0.5)."""
    rng = np.random.default_rng(500 + L)
    K = 2048
    rows = []
    for C in (63, 64, 65):
        x = (rng.random(L) * 0.5).astype(np.float32)
        pos = rng.permutation(L)
        above = K - 40
        x[pos[:above]] = (1000.0 + np.arange(above)).astype(np.float32)
        x[pos[above:above + C]] = (50.0 + (np.arange(C) % 8) / 64.0).astype(np.float32)
        rows.append(x)
    x = np.stack(rows)
    R = len(rows)
    q_pos = np.full((R, 1), L - 1, dtype=np.int32)
    scores = torch.from_numpy(x).view(R, 1, L).cuda()
    idx = dsa.topk(scores, torch.from_numpy(q_pos).cuda(), K)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for r in range(R):
        want = oracle.topk_row(x[r], L - 1, K)
        assert np.array_equal(got[r, 0], want), f"L={L} cluster {63 + r}"
