"""Oracle for hybrid prefill (TEST INFRASTRUCTURE ONLY; numpy, fp32).

Notation: Hq query heads, Hkv KV heads, G = Hq/Hkv, query head h reads KV
head h // G. S tokens, head dim d, block size B, n_b = ceil(S/B) blocks,
indexer rank r, k = number of top-scored candidate blocks kept in addition to
the sink block 0 and the diagonal block, w = sliding window.

Steps, in the order the pages give them:

1. Streaming heads ("化繁为简，被低估的 SWA" in the Synced RTPurbo article:
   most heads keep only nearby tokens): query i attends keys
   i - w < j <= i.
2. Retrieval heads (RTPurboV2 article, paragraph on the low-rank projector
   that maps D to r = 16; aitop.news summary: a 16-dim indexer finds the
   tokens that matter, then exact attention runs on that set):
   a. project every key, k^_j = P_k k_j;
   b. project every query, q~_i = P_q q_i, and average per query block,
      q-_qb = mean_{i in qb} q~_i;
   c. score each candidate block 1 <= kb <= qb-1 by
      sc(qb, kb) = max_{j in kb} q-_qb . k^_j;
   d. keep the k best candidates (ties: lower block index first);
   e. Sel(qb) = {0} u top-k u {qb};
   f. query i in block qb attends every key j <= i of the selected blocks.
3. Attention over a key set J_i (both head kinds): s_j = scale * q_i . k_j,
   lse_i = log sum_{j in J_i} exp(s_j), p_j = exp(s_j - lse_i),
   o_i = sum_j p_j v_j. The softmax is kept exact; only the key set shrinks.

Variant (RTPurboV2 article, paragraph on the Qwen3-Coder-30B-A3B setup):
the window may differ per streaming head (some are 8192), and retrieval
heads may use full attention in prefill, J_i = {j <= i}, while the key
clustering (the block centroids of step 2a's projected keys) is still
produced for decode.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional

import numpy as np

from .numerics import bf16_to_f32, f32_to_bf16

F32 = np.float32


def project_keys(k_g: np.ndarray, p_k: np.ndarray) -> np.ndarray:
    """Step 2a: k^_j = P_k k_j for every key. [S,d] x [r,d] -> [S,r]."""
    return (k_g.astype(F32) @ p_k.astype(F32).T).astype(F32)


def query_block_means(q_h: np.ndarray, p_q: np.ndarray, B: int) -> np.ndarray:
    """Step 2b, literal order: project each query, then average per block.

    A partial last block averages the queries it has. [S,d] -> [n_b,r].
    """
    S = q_h.shape[0]
    n_b = -(-S // B)
    qt = (q_h.astype(F32) @ p_q.astype(F32).T).astype(F32)
    out = np.empty((n_b, p_q.shape[0]), dtype=F32)
    for b in range(n_b):
        out[b] = qt[b * B:min(S, (b + 1) * B)].mean(axis=0, dtype=F32)
    return out


def block_score_row(qbar_row: np.ndarray, khat: np.ndarray, qb: int,
                    B: int) -> np.ndarray:
    """Step 2c for one query block: scores of candidates kb = 1 .. qb-1.

    Candidate blocks lie strictly before the diagonal block, so they are
    always full blocks. Returns an array of length max(qb-1, 0).
    """
    if qb < 2:
        return np.zeros(0, dtype=F32)
    dots = (khat[B:qb * B].astype(F32) @ qbar_row.astype(F32)).astype(F32)
    return dots.reshape(qb - 1, B).max(axis=1)


def select_row(sc: np.ndarray, qb: int, k: int):
    """Steps 2d-2e for one query block.

    Returns (Sel ascending, s_k, s_{k+1}) where s_k is the k-th largest
    candidate score (NaN when fewer than k candidates or k = 0) and s_{k+1}
    the next one (NaN when fewer than k+1 candidates).
    """
    cand = np.arange(1, max(qb, 1), dtype=np.int64)
    assert len(sc) == len(cand)
    if len(cand):
        order = np.lexsort((cand, -sc))          # -score, then block index
        top = cand[order[:k]]
        s_k = float(sc[order[k - 1]]) if 1 <= k <= len(cand) else math.nan
        s_k1 = float(sc[order[k]]) if k + 1 <= len(cand) else math.nan
    else:
        top = cand
        s_k = s_k1 = math.nan
    sel = np.unique(np.concatenate([[0], top, [qb]]).astype(np.int64))
    return sel, s_k, s_k1


def retrieval_selection(q_h: np.ndarray, k_g: np.ndarray, p_q: np.ndarray,
                        p_k: np.ndarray, B: int, k: int,
                        rows: Optional[Iterable[int]] = None):
    """Steps 2a-2e for one retrieval head. q_h, k_g are fp32 [S,d].

    Returns (sel: dict qb -> ascending block ids, kth: dict qb -> (s_k,
    s_{k+1}), khat [S,r], qbar [n_b,r]).
    """
    khat = project_keys(k_g, p_k)
    qbar = query_block_means(q_h, p_q, B)
    n_b = qbar.shape[0]
    rows = range(n_b) if rows is None else rows
    sel, kth = {}, {}
    for qb in rows:
        sc = block_score_row(qbar[qb], khat, qb, B)
        s, a, b = select_row(sc, qb, k)
        sel[qb], kth[qb] = s, (a, b)
    return sel, kth, khat, qbar


def block_centroids(khat: np.ndarray, B: int) -> np.ndarray:
    """Per-block mean of projected keys (clustering input for decode)."""
    S = khat.shape[0]
    n_b = -(-S // B)
    out = np.empty((n_b, khat.shape[1]), dtype=F32)
    for b in range(n_b):
        out[b] = khat[b * B:min(S, (b + 1) * B)].mean(axis=0, dtype=F32)
    return out


def swa_keys(i: int, w: int) -> np.ndarray:
    """Step 1: keys of query i under window w: i - w < j <= i."""
    return np.arange(max(0, i - w + 1), i + 1, dtype=np.int64)


def selected_keys(sel: np.ndarray, i: int, B: int, S: int) -> np.ndarray:
    """Step 2f: tokens of the selected blocks that are not after i."""
    parts = [np.arange(b * B, min(S, (b + 1) * B), dtype=np.int64)
             for b in sel]
    j = np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)
    return j[j <= i]


def head_window(window, h: int) -> int:
    """Window of streaming head h: one window for all heads, or head h's
    entry of a per-head sequence (RTPurboV2 article, Qwen3-Coder-30B-A3B
    paragraph: streaming heads use SWA, some with 8192)."""
    if np.ndim(window) == 0:
        return int(window)
    return int(np.asarray(window)[h])


def causal_block_keys(rows: np.ndarray):
    """Keys of a full (causal) head for a run of queries: every j <= i."""
    union = np.arange(0, int(rows[-1]) + 1, dtype=np.int64)
    return union, union[None, :] <= rows[:, None]


def swa_block_keys(rows: np.ndarray, w: int):
    """Step 1 for a run of consecutive queries: (union of keys, membership).

    membership[r, c] is the predicate i - w < j <= i for i = rows[r],
    j = union[c].
    """
    lo = max(0, int(rows[0]) - w + 1)
    union = np.arange(lo, int(rows[-1]) + 1, dtype=np.int64)
    i = rows[:, None]
    j = union[None, :]
    return union, (j <= i) & (j > i - w)


def retrieval_block_keys(rows: np.ndarray, sel: np.ndarray, B: int, S: int):
    """Step 2f for the queries of one block: (union of keys, membership).

    union holds every token of the selected blocks; membership[r, c] is
    j <= i for i = rows[r], j = union[c].
    """
    parts = [np.arange(b * B, min(S, (b + 1) * B), dtype=np.int64)
             for b in sel]
    union = np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)
    return union, union[None, :] <= rows[:, None]


def attend(q_rows: np.ndarray, k_keys: np.ndarray, v_keys: np.ndarray,
           member: np.ndarray, scale: float):
    """Step 3 for a batch of queries over a shared list of keys.

    member[r, c] says whether key c belongs to query r's set J; keys outside
    the set get exp(-inf) = 0, so each row is exactly the per-query
    definition. Returns (O [n,d] fp32, lse [n] fp32, natural log).
    """
    s = (q_rows.astype(F32) @ k_keys.astype(F32).T).astype(F32) * F32(scale)
    s = np.where(member, s, F32(-np.inf)).astype(F32)
    m = s.max(axis=1, keepdims=True)
    lse = (m[:, 0] + np.log(np.exp(s - m, dtype=F32).sum(axis=1, dtype=F32),
                            dtype=F32)).astype(F32)
    p = np.exp(s - lse[:, None], dtype=F32)
    o = (p @ v_keys.astype(F32)).astype(F32)
    return o, lse


def hybrid_prefill(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray,
                   is_retrieval, window: int, p_q: np.ndarray,
                   p_k: np.ndarray, block: int, top_k: int,
                   scale: Optional[float] = None, sel_override=None,
                   heads: Optional[Iterable[int]] = None,
                   query_blocks: Optional[Iterable[int]] = None,
                   sel_rows: Optional[Iterable[int]] = None,
                   retrieval_full: bool = False) -> dict:
    """Headwise hybrid prefill of one layer.

    window: one window for every streaming head, or a sequence of Hq
    windows (entries of retrieval heads unused). retrieval_full: retrieval
    heads attend every key j <= i (no selection; centroids are still
    computed when p_k is given).

    q_bits [Hq,S,d], k_bits/v_bits [Hkv,S,d]: bf16 storage (uint16).
    is_retrieval [Hq]: nonzero marks a retrieval head; p_q/p_k [n_ret,r,d]
    belong to the retrieval heads in ascending head order.
    sel_override: optional dict rho -> {qb: ascending block ids} replacing
    steps 2a-2e, so attention can be compared under an identical selection.
    heads / query_blocks restrict which outputs are computed (others stay
    NaN); sel_rows restricts which selection rows are computed (default: all
    rows, or the query_blocks when given).

    Returns out (fp32 [Hq,S,d]), out_bf16 (uint16), lse (fp32 [Hq,S]) (all
    three None when no output rows are requested: heads or query_blocks
    empty; out_bf16 holds the bf16 NaN pattern outside the computed rows), and
    for retrieval heads sel [n_ret,n_b,k+2] (ascending, -1 padded),
    sel_count [n_ret,n_b], kth [n_ret,n_b,2], centroids [n_ret,n_b,r].
    """
    Hq, S, d = q_bits.shape
    Hkv = k_bits.shape[0]
    G = Hq // Hkv
    B = block
    n_b = -(-S // B)
    mask = np.asarray(is_retrieval).astype(bool)
    ret_heads = [h for h in range(Hq) if mask[h]]
    rho_of = {h: i for i, h in enumerate(ret_heads)}
    scale = 1.0 / math.sqrt(d) if scale is None or scale <= 0 else scale
    heads = range(Hq) if heads is None else list(heads)
    qblocks = list(range(n_b)) if query_blocks is None else list(query_blocks)
    if sel_rows is None:
        sel_rows = qblocks
    sel_rows = sorted(set(sel_rows))

    # Output arrays only when some output row is asked for: a selection-only
    # call at long S would otherwise fill (and round) Hq*S*d unused values.
    want_out = len(heads) > 0 and len(qblocks) > 0
    out = np.full((Hq, S, d), np.nan, dtype=F32) if want_out else None
    lse = np.full((Hq, S), np.nan, dtype=F32) if want_out else None
    out_bf16 = (np.full((Hq, S, d), 0x7FC0, dtype=np.uint16) if want_out
                else None)
    n_ret = len(ret_heads)
    sel_arr = np.full((n_ret, n_b, top_k + 2), -1, dtype=np.int32)
    sel_cnt = np.zeros((n_ret, n_b), dtype=np.int32)
    kth = np.full((n_ret, n_b, 2), np.nan, dtype=F32)
    cents = np.full((n_ret, n_b, p_k.shape[1] if n_ret else 0), np.nan,
                    dtype=F32)
    kv_cache = {}

    def kv(g):
        if g not in kv_cache:
            kv_cache.clear()
            kv_cache[g] = (bf16_to_f32(k_bits[g]),
                           bf16_to_f32(v_bits[g]) if want_out else None)
        return kv_cache[g]

    for h in heads:
        g = h // G
        kf, vf = kv(g)
        qf = bf16_to_f32(q_bits[h])
        if mask[h] and retrieval_full:
            rho = rho_of[h]
            if p_k is not None and n_ret:
                cents[rho] = block_centroids(project_keys(kf, p_k[rho]), B)
        elif mask[h]:
            rho = rho_of[h]
            if sel_override is not None:
                sel = sel_override[rho]
            else:
                sel, kk, khat, _ = retrieval_selection(
                    qf, kf, p_q[rho], p_k[rho], B, top_k, rows=sel_rows)
                for qb, (a, b) in kk.items():
                    kth[rho, qb] = (a, b)
                cents[rho] = block_centroids(khat, B)
            for qb, s in sel.items():
                sel_arr[rho, qb, :len(s)] = s
                sel_cnt[rho, qb] = len(s)
        for qb in qblocks:
            rows = np.arange(qb * B, min(S, (qb + 1) * B))
            if mask[h] and retrieval_full:
                union, member = causal_block_keys(rows)
            elif mask[h]:
                union, member = retrieval_block_keys(rows, sel[qb], B, S)
            else:
                union, member = swa_block_keys(rows, head_window(window, h))
            o, l = attend(qf[rows], kf[union], vf[union], member, scale)
            out[h, rows] = o
            out_bf16[h, rows] = f32_to_bf16(o)
            lse[h, rows] = l
    return dict(out=out, out_bf16=out_bf16, lse=lse, sel=sel_arr,
                sel_count=sel_cnt, kth=kth, centroids=cents,
                retrieval_heads=np.array(ret_heads, dtype=np.int64))
