"""Pins of the clustering oracle (oracle/cluster.py) against what does not
depend on it: a library k-means, hand-worked tiny cases, the k-means
objective, planted structure known by construction, the block decode oracle
(pinned on its own), and an fp64 brute force of the clustered decode step.
CPU only.
"""
import math

import numpy as np
import pytest

import oracle
import oracle.cluster as oc
from tests.test_oracle_pins import _decode, _f32, _run_dec

F64 = np.float64


# ------------------------------------------------------------- Lloyd steps
def _lloyd(x, cents, T):
    for _ in range(T):
        a, cents, cnt = oc.lloyd_step(x, cents)
    return a, cents, cnt


@pytest.mark.parametrize("T", [1, 2, 3])
def test_lloyd_matches_sklearn_kmeans(T):
    # scikit-learn's Lloyd k-means (fp64, n_init=1, the given seeds, tol=0)
    # run for T iterations: its centres equal ours after T steps, and its
    # labels (one more assignment against the final centres) equal the
    # assignment of our step T+1. No cluster empties on the way, so its
    # empty-cluster relocation never runs.
    from sklearn.cluster import KMeans
    rng = np.random.default_rng(T)
    B, m = 64, 41
    x = rng.standard_normal((B * (m - 1), 16)) * rng.uniform(0.5, 2.0, 16)
    init = np.full((m, 16), np.nan)
    for c in range(1, m):
        init[c] = x[(c - 1) * B:c * B].mean(axis=0)
    a, cents, cnt = _lloyd(x, init.copy(), T)
    a_next, _, cnt_next = oc.lloyd_step(x, cents)
    assert (cnt[1:] > 0).all() and (cnt_next[1:] > 0).all()
    km = KMeans(n_clusters=m - 1, init=init[1:], n_init=1, max_iter=T,
                tol=0.0, algorithm="lloyd").fit(x)
    assert np.abs(km.cluster_centers_ - cents[1:]).max() < 1e-9
    assert np.array_equal(km.labels_ + 1, a_next)


def test_lloyd_brute_force_ties_and_empty_clusters():
    # points on a line (r = 2, second coordinate 0), worked by hand:
    # centroids c1 = (0,0), c2 = (4,0), c3 = (100,0) (no point near it)
    x = np.array([[0.0, 0], [1, 0], [2, 0], [3, 0], [4, 0], [-1, 0]])
    cents = np.array([[np.nan, np.nan], [0, 0], [4, 0], [100, 0]], F64)
    a, new, cnt = oc.lloyd_step(x, cents)
    # x = 2 is equidistant from c1 and c2: the lower index wins
    assert a.tolist() == [1, 1, 1, 2, 2, 1]
    assert cnt.tolist() == [0, 4, 2, 0]
    assert np.allclose(new[1], [(0 + 1 + 2 - 1) / 4, 0])
    assert np.allclose(new[2], [3.5, 0])
    # the empty cluster keeps its centroid
    assert new[3].tolist() == [100.0, 0.0]
    # and the same by explicit loops over every point and cluster
    for i, p in enumerate(x):
        d2 = [sum((p[j] - cents[c][j]) ** 2 for j in range(2))
              for c in range(1, 4)]
        best = min(range(3), key=lambda c: (d2[c], c))
        assert a[i] == best + 1


def test_kmeans_objective_never_increases():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64 * 30, 16))
    m = 31
    cents = np.full((m, 16), np.nan)
    for c in range(1, m):
        cents[c] = x[(c - 1) * 64:c * 64].mean(axis=0)
    prev = math.inf
    for _ in range(6):
        a, cents, _ = oc.lloyd_step(x, cents)
        inertia = float(((x - cents[a]) ** 2).sum())
        assert inertia <= prev + 1e-9
        prev = inertia


def _planted_keys(C, d=128, r=16, B=64, n_recent=2, seed=3):
    """Keys whose projections x = P_k k are planted: topic c has direction
    u_c (orthonormal) and norm s_c in [3, 12]; 70% of block c's tokens are
    topic c, the rest random other topics, so block c's mean is nearest to
    topic c and the topics are recovered after one step. P_k has
    orthonormal rows, and k = P_k^T x + (a component P_k ignores)."""
    rng = np.random.default_rng(seed)
    qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    p_k = qm[:r].astype(np.float32)
    u, _ = np.linalg.qr(rng.standard_normal((r, r)))
    dirs = u[:C] * rng.uniform(3.0, 12.0, C)[:, None]      # C <= r
    L = B * (C + n_recent) + 5             # m = C + 1
    topic = np.full(L, -1)
    for c in range(C):
        t = np.where(rng.random(B) < 0.7, c, rng.integers(0, C, B))
        topic[B * (c + 1):B * (c + 2)] = t
    x = np.zeros((L, r))
    inner = topic >= 0
    x[inner] = dirs[topic[inner]] + 0.05 * rng.standard_normal((inner.sum(), r))
    k = x @ p_k.astype(F64) + 0.3 * rng.standard_normal((L, d)) @ \
        (np.eye(d) - p_k.T.astype(F64) @ p_k.astype(F64))
    return k, p_k, topic, L


def test_planted_topics_are_recovered():
    # Scattered topics of different norms, seeded by blocks that each hold
    # a majority of one topic: two steps must give every token its topic's
    # cluster, and each centroid the mean of its members (sums instead of
    # means, a wrong cluster range or wrong seeds break the recovery).
    import torch
    C = 12
    k, p_k, topic, L = _planted_keys(C)
    kb = torch.from_numpy(k.astype(np.float32)).to(torch.bfloat16)
    bits = kb.view(torch.int16).numpy().view(np.uint16)
    kc = bits[None, None]                                   # [1,1,L,d]
    res = oc.cluster_keys(kc, [L], [1], p_k[None], block=64, n_recent=2,
                          iters=2)
    m = res["m"][0]
    assert m == C + 1
    a = res["assign"][(0, 0)]
    assert np.array_equal(a, topic[64:64 * m] + 1)
    # each centroid is its topic's mean (within the planted noise)
    cents = res["cents"][(0, 0)]
    x = res["x"][(0, 0)]
    for c in range(1, m):
        assert np.allclose(cents[c], x[a == c].mean(0))


def test_cluster_range_and_tables():
    # m = max(ceil(L/64) - n_recent, 1), worked by hand
    assert oc.cluster_count(64 * 10 + 5, 64, 2) == 9      # n_b 11
    assert oc.cluster_count(64 * 10, 64, 2) == 8          # n_b 10
    assert oc.cluster_count(64 * 10, 64, 1) == 9
    assert oc.cluster_count(130, 64, 2) == 1              # n_b 3: none
    assert oc.cluster_count(1, 64, 2) == 1
    # tables from an assignment, checked element by element
    rng = np.random.default_rng(1)
    m = 7
    assign = rng.integers(1, m, 64 * 6)
    off, mem = oc.group_members(assign, m, 64)
    assert off[0] == 0 and off[1] == 0 and off[m] == len(assign)
    for c in range(1, m):
        want = [64 + i for i in range(len(assign)) if assign[i] == c]
        assert mem[off[c]:off[c + 1]].tolist() == want
    # with no steps the clusters are the blocks: tokens 64 .. 64m-1 in order
    x = _decode(1, 64 * 10 + 5, Hq=2, Hkv=1, d=64, ret=(1,), window=8,
                top_k=3)
    res = oc.cluster_keys(x["kb"], x["cache_len"], x["is_retrieval"],
                          x["p_k"], iters=0)
    m = res["m"][0]
    assert m == 9
    assert res["members"][(0, 0)].tolist() == list(range(64, 64 * 9))
    assert res["offsets"][(0, 0)].tolist() == [0, 0] + \
        [64 * c for c in range(1, 9)]


def test_cluster_seeds_equal_decode_centroids():
    # the seeds are the block centroids of the block decode (pinned on its
    # own): mean over the block of P_k k
    x = _decode(2, 64 * 9 + 7, Hq=4, Hkv=2, d=64, ret=(0, 3), window=8,
                top_k=3, lens=[64 * 9 + 7, 64 * 5])
    res = oc.cluster_keys(x["kb"], x["cache_len"], x["is_retrieval"],
                          x["p_k"], iters=0)
    k = _f32(x["kb"])
    for b, L in enumerate(x["cache_len"]):
        m = res["m"][b]
        for rho, h in enumerate((0, 3)):
            dc = oracle.decode_centroids(k[b, h // 2], x["p_k"][rho], 64,
                                         int(L) // 64)
            cents = res["cents"][(b, rho)]
            for c in range(1, m):
                assert np.allclose(cents[c], dc[c], rtol=1e-5, atol=1e-6)


# --------------------------------------------------------- clustered decode
def test_clustered_decode_with_block_clusters_equals_block_decode():
    lens = [64 * 30 + 17, 64 * 12, 200, 64 * 7 + 1]
    x = _decode(4, max(lens), Hq=4, Hkv=2, d=64, ret=(0, 3), window=40,
                top_k=5, lens=lens, seed=2)
    cl = oc.cluster_keys(x["kb"], x["cache_len"], x["is_retrieval"],
                         x["p_k"], iters=0)
    # the block decode scores fp32 block centroids: hand those over
    k = _f32(x["kb"])
    for b, L in enumerate(lens):
        for rho, h in enumerate((0, 3)):
            dc = oracle.decode_centroids(k[b, h // 2], x["p_k"][rho], 64,
                                         L // 64)
            m = cl["m"][b]
            cl["cents"][(b, rho)] = dc[:m] if m > 1 else dc[:1]
    got = oc.clustered_decode(x["qb"], x["kb"], x["vb"], x["cache_len"],
                              x["is_retrieval"], x["window"], x["p_q"],
                              x["p_k"], 64, x["top_k"], cl)
    want = _run_dec(x)
    assert np.array_equal(got["out"], want["out"])
    for (b, rho), sel in got["sel"].items():
        row = want["sel"][b, rho]
        assert sel.tolist() == row[row >= 0].tolist()


def test_clustered_decode_fp64_brute_force():
    # Random cluster tables over blocks 1..m-1, the cache grown after the
    # clustering (so blocks m .. n_b-3 are ordinary candidates), one empty
    # cluster whose (stale) centroid scores highest, a later block that
    # scores high, and two clusters with equal centroids at the cut. The
    # kept set and the output are rebuilt here in fp64 with explicit loops.
    rng = np.random.default_rng(11)
    L0 = 64 * 20 + 3                         # length when clustered
    L = L0 + 64 * 4 + 10                     # length now
    x = _decode(1, L, Hq=2, Hkv=1, d=64, ret=(1,), window=8, top_k=6,
                seed=5)
    m = oc.cluster_count(L0, 64, 2)          # 19
    n_tok = 64 * (m - 1)
    assign = rng.integers(1, m, n_tok)
    assign[assign == 4] = 5                  # cluster 4 is empty
    off, mem = oc.group_members(assign, m, 64)
    qf = _f32(x["qb"])[0, 1].astype(F64)
    qt = x["p_q"][0].astype(F64) @ qf
    u = qt / np.linalg.norm(qt)
    cents = 0.01 * rng.standard_normal((m, 16))
    cents[[1, 2, 3, 5]] += 2 * u             # clearly kept
    cents[4] = 50 * u                        # empty: would score highest
    cents[7] = cents[9] = 0.5 * u            # tie at the cut: 7 is kept
    cents = cents.astype(np.float32).astype(F64)
    cl = dict(m=np.array([m]), cents={(0, 0): cents},
              offsets={(0, 0): off}, members={(0, 0): mem})
    k, v = _f32(x["kb"])[0, 0].astype(F64), _f32(x["vb"])[0, 0].astype(F64)
    # plant a high-scoring later block (block m + 1)
    blk = m + 1
    kf = _f32(x["kb"])
    kb_new = x["kb"].copy()
    dirk = np.linalg.lstsq(x["p_k"][0].astype(F64), qt, rcond=None)[0]
    import torch
    rows = (kf[0, 0, 64 * blk:64 * blk + 64] + 0.5 * dirk / np.abs(dirk).max()
            ).astype(np.float32)
    kb_new[0, 0, 64 * blk:64 * blk + 64] = torch.from_numpy(rows).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    x["kb"] = kb_new
    k = _f32(x["kb"])[0, 0].astype(F64)
    n_b = -(-L // 64)
    top_k = 6
    # brute force: candidates 1 .. n_b-3
    cand = []
    for c in range(1, n_b - 2):
        if c < m:
            if off[c + 1] == off[c]:
                continue
            cent = cents[c]
        else:
            cent = (k[64 * c:64 * c + 64] @ x["p_k"][0].astype(F64).T).mean(0)
        cand.append((-(float(cent @ qt)), c))
    cand.sort()
    top = sorted(c for _, c in cand[:top_k])
    assert blk in top and 4 not in top and (7 in top) != (9 in top)
    keep = [0] + top + [n_b - 2, n_b - 1]
    toks = []
    for c in keep:
        if 1 <= c < m:
            toks += [int(t) for t in range(64, 64 * m) if assign[t - 64] == c]
        else:
            toks += list(range(64 * c, min(L, 64 * c + 64)))
    toks = sorted(toks)
    s = (k[toks] @ qf) / math.sqrt(64)
    p = np.exp(s - s.max())
    o = (p / p.sum()) @ v[toks]
    got = oc.clustered_decode(x["qb"], x["kb"], x["vb"], x["cache_len"],
                              x["is_retrieval"], x["window"], x["p_q"],
                              x["p_k"], 64, top_k, cl)
    assert got["sel"][(0, 0)].tolist() == keep
    assert got["keys"][(0, 0)].tolist() == toks
    assert np.abs(got["out"][0, 1] - o).max() < 1e-5
