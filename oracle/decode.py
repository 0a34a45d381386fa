"""Oracle for hybrid decode (TEST INFRASTRUCTURE ONLY; numpy, fp32).

The RTPurboV2 article (paragraphs on clustering in the low-rank space and on
the Qwen3-Coder recipe: K-cache clustering, sparse retrieval heads during
decode, SWA elsewhere) describes decode as: group the cached keys in the
projected space, score the groups with the projected query, and attend
exactly to the chosen groups. This library's reading, written out here:

* groups are contiguous B-token blocks; for each full block kb the centroid
  is c_kb = mean_{j in kb} P_k k_j (project each key, then average);
* the new query (at position L-1, L = cache length counting it) is projected,
  q~ = P_q q, and scores candidates 1 .. n_b - n_recent - 1 by q~ . c_kb;
* Sel = {0} u top-k u {the last n_recent blocks} (ties: lower block index);
  a short cache where |candidates| <= k keeps every block;
* retrieval heads attend every cached token of the selected blocks;
  streaming heads attend the last w tokens, L-w <= j <= L-1;
* the softmax/PV step is the same exact attention as in prefill.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional

import numpy as np

from .numerics import bf16_to_f32, f32_to_bf16
from .prefill import attend

F32 = np.float32


def decode_centroids(k_seq: np.ndarray, p_k: np.ndarray, B: int,
                     n_full: int) -> np.ndarray:
    """c_kb = mean over the B keys of block kb of P_k k_j, full blocks only.

    k_seq fp32 [>= n_full*B, d] -> [n_full, r].
    """
    proj = (k_seq[:n_full * B].astype(F32) @ p_k.astype(F32).T).astype(F32)
    out = np.empty((n_full, p_k.shape[0]), dtype=F32)
    for b in range(n_full):
        out[b] = proj[b * B:(b + 1) * B].mean(axis=0, dtype=F32)
    return out


def decode_select(q_tilde: np.ndarray, cents: np.ndarray, n_b: int, k: int,
                  n_recent: int):
    """Block choice for one (sequence, retrieval head).

    Returns (Sel ascending, s_k, s_{k+1}); s_k / s_{k+1} as in prefill.
    """
    n_c = max(n_b - n_recent - 1, 0)
    cand = np.arange(1, 1 + n_c, dtype=np.int64)
    if n_c:
        sc = (cents[cand].astype(F32) @ q_tilde.astype(F32)).astype(F32)
        order = np.lexsort((cand, -sc))
        top = cand[order[:k]]
        s_k = float(sc[order[k - 1]]) if 1 <= k <= n_c else math.nan
        s_k1 = float(sc[order[k]]) if k + 1 <= n_c else math.nan
    else:
        top = cand
        s_k = s_k1 = math.nan
    recent = np.arange(n_b - n_recent, n_b, dtype=np.int64)
    sel = np.concatenate([[0], top, recent]).astype(np.int64)
    sel = np.unique(sel[sel >= 0])
    return sel, s_k, s_k1


def hybrid_decode(q_bits: np.ndarray, kc_bits: np.ndarray,
                  vc_bits: np.ndarray, cache_len, is_retrieval, window: int,
                  p_q: np.ndarray, p_k: np.ndarray, block: int, top_k: int,
                  n_recent: int = 2, scale: Optional[float] = None,
                  seqs: Optional[Iterable[int]] = None,
                  sel_override: Optional[dict] = None) -> dict:
    """One decode step for a batch.

    q_bits [Bn,Hq,d]; kc_bits/vc_bits [Bn,Hkv,Lmax,d] (bf16 storage);
    cache_len [Bn] counts the new token. sel_override: optional dict
    (b, rho) -> ascending block ids that replaces the block choice of that
    (sequence, retrieval head), so attention can be compared under an
    identical selection (centroids are still computed). Returns out fp32
    [Bn,Hq,d],
    out_bf16, lse [Bn,Hq], sel [Bn,n_ret,top_k+1+n_recent] (ascending,
    -1 padded), sel_count [Bn,n_ret], kth [Bn,n_ret,2],
    centroids dict (b, rho) -> [n_full, r].
    """
    Bn, Hq, d = q_bits.shape
    Hkv = kc_bits.shape[1]
    G = Hq // Hkv
    B = block
    mask = np.asarray(is_retrieval).astype(bool)
    ret_heads = [h for h in range(Hq) if mask[h]]
    n_ret = len(ret_heads)
    scale = 1.0 / math.sqrt(d) if scale is None or scale <= 0 else scale
    seqs = range(Bn) if seqs is None else list(seqs)

    out = np.full((Bn, Hq, d), np.nan, dtype=F32)
    lse = np.full((Bn, Hq), np.nan, dtype=F32)
    width = top_k + 1 + n_recent
    sel_arr = np.full((Bn, n_ret, width), -1, dtype=np.int32)
    sel_cnt = np.zeros((Bn, n_ret), dtype=np.int32)
    kth = np.full((Bn, n_ret, 2), np.nan, dtype=F32)
    cents = {}
    for b in seqs:
        L = int(cache_len[b])
        n_b = -(-L // B)
        n_full = L // B
        for g in range(Hkv):
            kf = bf16_to_f32(kc_bits[b, g, :L])
            vf = bf16_to_f32(vc_bits[b, g, :L])
            for h in range(g * G, (g + 1) * G):
                qf = bf16_to_f32(q_bits[b, h])
                if mask[h]:
                    rho = ret_heads.index(h)
                    c = decode_centroids(kf, p_k[rho], B, n_full)
                    cents[(b, rho)] = c
                    if sel_override is not None and (b, rho) in \
                            sel_override:
                        sel = np.asarray(sel_override[(b, rho)],
                                         dtype=np.int64)
                        s_k = s_k1 = math.nan
                    else:
                        qt = (p_q[rho].astype(F32) @ qf).astype(F32)
                        sel, s_k, s_k1 = decode_select(qt, c, n_b, top_k,
                                                       n_recent)
                    sel_arr[b, rho, :len(sel)] = sel
                    sel_cnt[b, rho] = len(sel)
                    kth[b, rho] = (s_k, s_k1)
                    keys = np.concatenate(
                        [np.arange(x * B, min(L, (x + 1) * B)) for x in sel])
                else:
                    keys = np.arange(max(0, L - window), L)
                member = np.ones((1, len(keys)), dtype=bool)
                o, l = attend(qf[None, :], kf[keys], vf[keys], member, scale)
                out[b, h] = o[0]
                lse[b, h] = l[0]
    return dict(out=out, out_bf16=f32_to_bf16(out), lse=lse, sel=sel_arr,
                sel_count=sel_cnt, kth=kth, centroids=cents,
                retrieval_heads=np.array(ret_heads, dtype=np.int64))
