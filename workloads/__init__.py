"""Seeded synthetic inputs for headwise hybrid attention.

This module only draws data. It holds none of the attention method's
arithmetic (no projection, scoring, selection or softmax), so both the CPU
oracle and the HIP path can take their inputs from it without sharing any
computation.

Recipe (the pages measure on real-model prefills and name no dataset; these
inputs stand in for them):

* Q/K/V of one attention layer are drawn N(0, 1) in fp32 and rounded to bf16
  (round-to-nearest-even, via torch's dtype cast).
* Retrieval heads are ``sorted(default_rng(seed).choice(Hq, n_ret,
  replace=False))`` unless a workload fixes them.
* The indexer projections P_q, P_k are drawn N(0, sd=1/sqrt(d)) in fp32 with
  shape [n_ret, r, d], independently per retrieval head.
* "Needle" workloads: per KV head g a unit direction u_g; 32 key blocks drawn
  without replacement from blocks 1 .. n_b/2-1 get K rows N(0,1) + 2 u_g, and
  every query row at position >= S/2 of each query head of group g gets
  + 2 u_g, so that late queries correlate with a few early key blocks.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class PrefillWorkload:
    name: str
    S: int
    Hq: int
    Hkv: int
    d: int
    n_ret: int
    window: int
    r: int
    block: int
    top_k: int
    needles: int = 0
    seed: int = 0
    retrieval_heads: Optional[Sequence[int]] = None

    @property
    def n_blocks(self) -> int:
        return -(-self.S // self.block)


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    batch: int
    L: int
    Hq: int
    Hkv: int
    d: int
    n_ret: int
    window: int
    r: int
    block: int
    top_k: int
    n_recent: int = 2
    seed: int = 0
    retrieval_heads: Optional[Sequence[int]] = None


# The five workloads of this library's benchmark, by what they are.
TINY = PrefillWorkload("tiny_2k_4q1kv", S=2048, Hq=4, Hkv=1, d=128, n_ret=1,
                       window=256, r=16, block=64, top_k=8,
                       retrieval_heads=(0,))
PREFILL_32K = PrefillWorkload("prefill_32k_qwen3_30b_a3b_layer", S=32768,
                              Hq=32, Hkv=4, d=128, n_ret=5, window=8192,
                              r=16, block=64, top_k=64)
PREFILL_128K = PrefillWorkload("prefill_128k_qwen3_30b_a3b_layer_needles",
                               S=131072, Hq=32, Hkv=4, d=128, n_ret=5,
                               window=8192, r=16, block=64, top_k=128,
                               needles=32)
PREFILL_1M = PrefillWorkload("prefill_1m_all_sparse_needles", S=1 << 20,
                             Hq=32, Hkv=4, d=128, n_ret=23, window=8192,
                             r=16, block=64, top_k=256, needles=32)
DECODE_32x256K = DecodeWorkload("decode_b32_256k_cache", batch=32, L=1 << 18,
                                Hq=32, Hkv=4, d=128, n_ret=5, window=8192,
                                r=16, block=64, top_k=64, n_recent=2)

PREFILL_WORKLOADS = {w.name: w for w in (TINY, PREFILL_32K, PREFILL_128K,
                                         PREFILL_1M)}


def retrieval_heads_for(Hq: int, n_ret: int, seed: int,
                        fixed: Optional[Sequence[int]] = None) -> np.ndarray:
    """Indices of the retrieval query heads, ascending."""
    if fixed is not None:
        return np.array(sorted(fixed), dtype=np.int64)
    rng = np.random.default_rng(seed)
    return np.array(sorted(rng.choice(Hq, n_ret, replace=False)),
                    dtype=np.int64)


def head_mask(Hq: int, heads: Sequence[int]) -> np.ndarray:
    m = np.zeros(Hq, dtype=np.uint8)
    m[list(heads)] = 1
    return m


def draw_projections(n_ret: int, r: int, d: int, seed: int):
    """P_q, P_k ~ N(0, sd=1/sqrt(d)), fp32 [n_ret, r, d]."""
    rng = np.random.default_rng([seed, 0x5eed, 1])
    sd = 1.0 / math.sqrt(d)
    p_q = rng.normal(0.0, sd, size=(n_ret, r, d)).astype(np.float32)
    p_k = rng.normal(0.0, sd, size=(n_ret, r, d)).astype(np.float32)
    return p_q, p_k


def _needle_plan(S: int, Hkv: int, d: int, block: int, n_needles: int,
                 seed: int):
    rng = np.random.default_rng([seed, 0x5eed, 2])
    n_b = -(-S // block)
    hi = n_b // 2  # candidate blocks 1 .. n_b/2 - 1
    dirs, blocks = [], []
    for _ in range(Hkv):
        u = rng.normal(size=d)
        u = (u / np.linalg.norm(u)).astype(np.float32)
        cand = np.arange(1, max(hi, 1))
        take = min(n_needles, len(cand))
        b = np.sort(rng.choice(cand, take, replace=False)) if take else \
            np.zeros(0, dtype=np.int64)
        dirs.append(u)
        blocks.append(b)
    return dirs, blocks


def _randn(shape, gen, device):
    return torch.randn(shape, generator=gen, device=device,
                       dtype=torch.float32)


def make_prefill(w: PrefillWorkload, device: str = "cpu") -> dict:
    """Draw one layer's inputs. Q [Hq,S,d], K/V [Hkv,S,d] bf16 on `device`.

    Per-head generation keeps the fp32 temporaries to one head at a time, so
    the 1M-token workload fits. Values depend on the device's generator
    (CPU and GPU streams differ); each caller hands the same tensors to both
    sides of a comparison.
    """
    heads = retrieval_heads_for(w.Hq, w.n_ret, w.seed, w.retrieval_heads)
    p_q, p_k = draw_projections(len(heads), w.r, w.d, w.seed)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(w.seed))
    G = w.Hq // w.Hkv
    dirs, nblocks = (_needle_plan(w.S, w.Hkv, w.d, w.block, w.needles, w.seed)
                     if w.needles else (None, None))
    q = torch.empty((w.Hq, w.S, w.d), dtype=torch.bfloat16, device=device)
    k = torch.empty((w.Hkv, w.S, w.d), dtype=torch.bfloat16, device=device)
    v = torch.empty((w.Hkv, w.S, w.d), dtype=torch.bfloat16, device=device)
    for h in range(w.Hq):
        x = _randn((w.S, w.d), gen, device)
        if dirs is not None:
            u = torch.from_numpy(dirs[h // G]).to(device)
            x[w.S // 2:] += 2.0 * u
        q[h] = x.to(torch.bfloat16)
    for g in range(w.Hkv):
        x = _randn((w.S, w.d), gen, device)
        if dirs is not None:
            u = torch.from_numpy(dirs[g]).to(device)
            for b in nblocks[g]:
                x[b * w.block:(b + 1) * w.block] += 2.0 * u
        k[g] = x.to(torch.bfloat16)
    for g in range(w.Hkv):
        v[g] = _randn((w.S, w.d), gen, device).to(torch.bfloat16)
    return dict(q=q, k=k, v=v, is_retrieval=head_mask(w.Hq, heads),
                retrieval_heads=heads, p_q=p_q, p_k=p_k, window=w.window,
                r=w.r, block=w.block, top_k=w.top_k,
                needle_blocks=nblocks, workload=w)


def make_decode(w: DecodeWorkload, device: str = "cpu",
                cache_len: Optional[Sequence[int]] = None,
                Lmax: Optional[int] = None) -> dict:
    """Draw one decode step's inputs.

    q [B,Hq,d]; k_cache/v_cache [B,Hkv,Lmax,d] (bf16, N(0,1), no needles);
    cache_len [B] int32 counts the new token, already appended at L-1.
    """
    heads = retrieval_heads_for(w.Hq, w.n_ret, w.seed, w.retrieval_heads)
    p_q, p_k = draw_projections(len(heads), w.r, w.d, w.seed)
    lens = np.full(w.batch, w.L, dtype=np.int32) if cache_len is None else \
        np.asarray(cache_len, dtype=np.int32)
    Lm = int(Lmax if Lmax is not None else lens.max())
    gen = torch.Generator(device=device)
    gen.manual_seed(int(w.seed))
    q = _randn((w.batch, w.Hq, w.d), gen, device).to(torch.bfloat16)
    kc = torch.empty((w.batch, w.Hkv, Lm, w.d), dtype=torch.bfloat16,
                     device=device)
    vc = torch.empty_like(kc)
    for b in range(w.batch):
        kc[b] = _randn((w.Hkv, Lm, w.d), gen, device).to(torch.bfloat16)
        vc[b] = _randn((w.Hkv, Lm, w.d), gen, device).to(torch.bfloat16)
    return dict(q=q, k_cache=kc, v_cache=vc, cache_len=lens,
                is_retrieval=head_mask(w.Hq, heads), retrieval_heads=heads,
                p_q=p_q, p_k=p_k, window=w.window, r=w.r, block=w.block,
                top_k=w.top_k, n_recent=w.n_recent, workload=w)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bf16 storage of a tensor as a host uint16 array (no arithmetic)."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(
        np.uint16)
