"""Oracle for semantic K-cache clustering and the clustered decode step
(TEST INFRASTRUCTURE ONLY; numpy; the clustering itself in fp64).

Source: "阿里RTPurboV2：Transformer再次崛起，百步训练实现10倍稀少把稳",
the paragraph on the synergy of the two compressions: once the projector has
filtered the high-frequency positional components, keys with related meaning
lie close together in the low-rank space and unrelated ones far apart, which
makes compression along the sequence by clustering possible (whole groups of
unrelated tokens are skipped); and the Qwen3-Coder recipe paragraph: the K
cache is clustered during prefill and decode runs sparsely on the retrieval
heads.

The pages name clustering but give no algorithm. This library's reading,
the plainest one that fits the rest of the decode recipe:

* points: the projected keys x_t = P_k k_t (r dims) of the candidate tokens
  of one (sequence, retrieval head), i.e. the tokens of blocks
  1 .. m-1 with m = max(n_b - n_recent, 1), n_b = ceil(L / B): the sink
  block and the last n_recent blocks are always attended and are not
  clustered;
* clusters: m - 1 of them, cluster c seeded by block c (its centroid starts
  as the mean of block c's projected keys), so the average cluster has B
  tokens and top_k clusters cost about what top_k blocks cost;
* k-means by Lloyd's algorithm, `iters` steps; one step assigns every point
  to the nearest centroid in Euclidean distance (ties: the lower cluster
  index), then moves every cluster that has members to the mean of its
  members; a cluster left without members keeps its centroid. With
  iters = 0 the clusters are the blocks themselves;
* members of a cluster are kept in ascending token order;
* decode: the projected query scores every non-empty cluster by
  q~ . centroid, and every later block (one that left the recent window
  after the clustering, c >= m) by its block centroid; the top_k candidates
  (ties: lower index) are kept together with the sink block and the last
  n_recent blocks; the head attends every member token of a kept cluster
  and every token of a kept block, exactly.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional

import numpy as np

from .numerics import bf16_to_f32, f32_to_bf16
from .prefill import attend
from .decode import decode_centroids

F32 = np.float32
F64 = np.float64


def cluster_count(L: int, block: int, n_recent: int) -> int:
    """m: clusters are 1 .. m-1 (blocks 1 .. m-1 seed them)."""
    n_b = -(-L // block)
    return max(n_b - n_recent, 1)


def project_keys64(k_rows: np.ndarray, p_k: np.ndarray) -> np.ndarray:
    """x_t = P_k k_t in fp64: [n, d] -> [n, r]."""
    return k_rows.astype(F64) @ p_k.astype(F64).T


def block_means(x: np.ndarray, m: int, block: int) -> np.ndarray:
    """Seeds: row c (1 <= c < m) is the mean of the projected keys of block
    c; x holds the candidate tokens block..block*m-1 in order. Row 0 unused
    (NaN)."""
    r = x.shape[1]
    out = np.full((m, r), np.nan, dtype=F64)
    for c in range(1, m):
        out[c] = x[(c - 1) * block:c * block].mean(axis=0)
    return out


def nearest_centroid(x: np.ndarray, cents: np.ndarray) -> np.ndarray:
    """Index (into cents) of the nearest centroid of every point, by squared
    Euclidean distance sum_i (x_i - c_i)^2; np.argmin takes the first
    minimum, i.e. ties go to the lower index. Points are taken in chunks
    only to bound memory."""
    out = np.empty(len(x), dtype=np.int64)
    chunk = max(1, 4_000_000 // max(1, cents.size))
    for s in range(0, len(x), chunk):
        xs = x[s:s + chunk]
        d2 = ((xs[:, None, :] - cents[None, :, :]) ** 2).sum(axis=2)
        out[s:s + chunk] = np.argmin(d2, axis=1)
    return out


def lloyd_step(x: np.ndarray, cents: np.ndarray):
    """One Lloyd step over the clusters 1..m-1 of `cents` ([m, r], row 0
    unused). Returns (assign [n] cluster ids, new cents [m, r], counts [m])."""
    m = cents.shape[0]
    assign = nearest_centroid(x, cents[1:]) + 1
    counts = np.bincount(assign, minlength=m)
    new = cents.copy()
    for c in range(1, m):
        if counts[c]:
            new[c] = x[assign == c].mean(axis=0)
    return assign, new, counts


def group_members(assign: np.ndarray, m: int, first_token: int):
    """Cluster tables from an assignment of tokens first_token, first_token+1,
    ...: offsets [m+1] (members of cluster c are members[offsets[c]:
    offsets[c+1]]; offsets[0] = offsets[1] = 0) and members ascending within
    each cluster."""
    counts = np.bincount(assign, minlength=m)[:m] if len(assign) else \
        np.zeros(m, dtype=np.int64)
    offsets = np.zeros(m + 1, dtype=np.int64)
    for c in range(1, m):
        offsets[c + 1] = offsets[c] + counts[c]
    members = np.empty(len(assign), dtype=np.int64)
    fill = offsets.copy()
    for i, c in enumerate(assign):
        members[fill[c]] = first_token + i
        fill[c] += 1
    return offsets, members


def cluster_keys(kc_bits: np.ndarray, cache_len, is_retrieval,
                 p_k: np.ndarray, block: int = 64, n_recent: int = 2,
                 iters: int = 1, seqs: Optional[Iterable[int]] = None,
                 init: Optional[dict] = None) -> dict:
    """Clusters the cached keys of every (sequence, retrieval head).

    kc_bits [Bn,Hkv,Lmax,d] bf16 storage; cache_len [Bn]; p_k [n_ret,r,d].
    init: optional dict (b, rho) -> [m, r] starting centroids (rows 1..m-1)
    in place of the block means. Returns dict with m [Bn] and, per
    (b, rho): cents [m, r] fp64, assign (cluster id of tokens B .. B*m-1),
    counts [m], offsets [m+1], members, x (the projected keys).
    """
    Bn, Hkv = kc_bits.shape[:2]
    mask = np.asarray(is_retrieval).astype(bool)
    Hq = len(mask)
    G = Hq // Hkv
    ret_heads = [h for h in range(Hq) if mask[h]]
    seqs = range(Bn) if seqs is None else list(seqs)
    res = dict(m=np.ones(Bn, dtype=np.int64), cents={}, assign={},
               counts={}, offsets={}, members={}, x={})
    for b in seqs:
        L = int(cache_len[b])
        m = cluster_count(L, block, n_recent)
        res["m"][b] = m
        for rho, h in enumerate(ret_heads):
            g = h // G
            kf = bf16_to_f32(kc_bits[b, g, block:block * m])
            x = project_keys64(kf, p_k[rho])
            if init is not None and (b, rho) in init:
                cents = np.asarray(init[(b, rho)], dtype=F64)[:m].copy()
            else:
                cents = block_means(x, m, block)
            assign = np.repeat(np.arange(1, m), block)
            counts = np.bincount(assign, minlength=m)
            for _ in range(iters if m > 1 else 0):
                assign, cents, counts = lloyd_step(x, cents)
            offsets, members = group_members(assign, m, block)
            key = (b, rho)
            res["cents"][key] = cents
            res["assign"][key] = assign
            res["counts"][key] = counts
            res["offsets"][key] = offsets
            res["members"][key] = members
            res["x"][key] = x
    return res


def clustered_select(q_tilde: np.ndarray, cent_of, valid_of, n_b: int,
                     k: int, n_recent: int):
    """Choice of one (sequence, retrieval head): candidates 1..n_b-n_recent-1
    that are valid (non-empty clusters and later blocks), scored in fp32 by
    q~ . centroid; top k by (score desc, index asc), or every valid
    candidate when there are at most k. Returns Sel ascending (with the
    sink and the recent blocks)."""
    n_c = max(n_b - n_recent - 1, 0)
    cand = np.array([c for c in range(1, 1 + n_c) if valid_of(c)],
                    dtype=np.int64)
    if len(cand) > k:
        cm = np.stack([cent_of(c) for c in cand]).astype(F32)
        sc = (cm @ q_tilde.astype(F32)).astype(F32)
        order = np.lexsort((cand, -sc))
        top = cand[order[:k]]
    else:
        top = cand
    recent = np.arange(n_b - n_recent, n_b, dtype=np.int64)
    sel = np.concatenate([[0], top, recent]).astype(np.int64)
    return np.unique(sel[sel >= 0])


def kept_tokens(sel, m: int, offsets, members, L: int, block: int):
    """Token ids attended for a choice `sel`: the members of kept clusters
    (1 <= c < m) and every token of kept blocks (the sink, later blocks,
    the recent blocks), ascending."""
    parts = [np.zeros(0, dtype=np.int64)]
    for c in sel:
        c = int(c)
        if 1 <= c < m:
            parts.append(np.asarray(members[offsets[c]:offsets[c + 1]]))
        else:
            parts.append(np.arange(c * block, min(L, (c + 1) * block)))
    return np.sort(np.concatenate(parts).astype(np.int64))


def clustered_decode(q_bits: np.ndarray, kc_bits: np.ndarray,
                     vc_bits: np.ndarray, cache_len, is_retrieval,
                     window: int, p_q: np.ndarray, p_k: np.ndarray,
                     block: int, top_k: int, clusters: dict,
                     n_recent: int = 2, scale: Optional[float] = None,
                     seqs: Optional[Iterable[int]] = None,
                     sel_override: Optional[dict] = None) -> dict:
    """One decode step whose retrieval heads choose among clusters.

    clusters: dict with m [Bn] and per (b, rho) cents [m, r] (rows 1..m-1
    used, taken at fp32 as a centroid table holds them), offsets [m+1] and
    members, as returned by cluster_keys (or read back from the library).
    cache_len may exceed the length the clusters were built at: blocks
    m .. n_b-n_recent-1 are then ordinary candidates with their block
    centroid. sel_override: dict (b, rho) -> ascending ids replacing the
    choice. Returns out fp32 [Bn,Hq,d], out_bf16, lse [Bn,Hq], sel (list
    per (b, rho)), and keys (the attended token ids per (b, rho)).
    """
    Bn, Hq, d = q_bits.shape
    Hkv = kc_bits.shape[1]
    G = Hq // Hkv
    B = block
    mask = np.asarray(is_retrieval).astype(bool)
    ret_heads = [h for h in range(Hq) if mask[h]]
    scale = 1.0 / math.sqrt(d) if scale is None or scale <= 0 else scale
    seqs = range(Bn) if seqs is None else list(seqs)
    out = np.full((Bn, Hq, d), np.nan, dtype=F32)
    lse = np.full((Bn, Hq), np.nan, dtype=F32)
    sels, keys_of = {}, {}
    for b in seqs:
        L = int(cache_len[b])
        n_b = -(-L // B)
        m = int(clusters["m"][b])
        for g in range(Hkv):
            kf = bf16_to_f32(kc_bits[b, g, :L])
            vf = bf16_to_f32(vc_bits[b, g, :L])
            for h in range(g * G, (g + 1) * G):
                qf = bf16_to_f32(q_bits[b, h])
                if mask[h]:
                    rho = ret_heads.index(h)
                    off = np.asarray(clusters["offsets"][(b, rho)])
                    mem = np.asarray(clusters["members"][(b, rho)])
                    cents = np.asarray(clusters["cents"][(b, rho)])
                    later = decode_centroids(kf, p_k[rho], B, L // B)

                    def cent_of(c):
                        return cents[c].astype(F32) if c < m else later[c]

                    def valid_of(c):
                        return c >= m or off[c + 1] > off[c]

                    if sel_override is not None and (b, rho) in sel_override:
                        sel = np.asarray(sel_override[(b, rho)], np.int64)
                    else:
                        qt = (p_q[rho].astype(F32) @ qf).astype(F32)
                        sel = clustered_select(qt, cent_of, valid_of, n_b,
                                               top_k, n_recent)
                    keys = kept_tokens(sel, m, off, mem, L, B)
                    sels[(b, rho)] = sel
                    keys_of[(b, rho)] = keys
                else:
                    keys = np.arange(max(0, L - window), L)
                member = np.ones((1, len(keys)), dtype=bool)
                o, l = attend(qf[None, :], kf[keys], vf[keys], member, scale)
                out[b, h] = o[0]
                lse[b, h] = l[0]
    return dict(out=out, out_bf16=f32_to_bf16(out), lse=lse, sel=sels,
                keys=keys_of, retrieval_heads=np.array(ret_heads, np.int64))
