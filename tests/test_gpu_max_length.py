"""GPU parity at the largest supported length: a prefill of S = 2^24 - 64
tokens, and a decode step on a cache of S + 1 tokens.

One KV head's K (and V^T) then fills a 4 GiB buffer descriptor up to its
last 16 KiB, every offset of the attention and indexer kernels takes its
largest value, and the fused scoring-and-selection kernel runs over 262 143
key blocks. One streaming head (window 4096) and one retrieval head share
the KV head. The oracle checks sampled selection rows (the first, around
S/2, the last and random ones, each up to 262 141 candidates) and the
outputs and LSE of sampled query blocks of both heads, under the GPU's
selection (identical to the oracle's except at logged ties). The decode
step chooses among 262 141 candidate blocks, attends a window of 8192 and
the chosen blocks, and is checked like every other decode test.
"""
import numpy as np
import pytest
import torch

import oracle
from tests import parity
from tests.test_gpu_decode import _wl as _dec_wl, check as dec_check
from workloads import PrefillWorkload, make_prefill, make_decode, bf16_bits

pytestmark = pytest.mark.gpu

S_MAX = (1 << 24) - 64


def _host_heads(t, heads):
    """uint16 host copy of t with only t[h], h in heads, filled."""
    arr = np.empty(tuple(t.shape), dtype=np.uint16)
    for h in heads:
        arr[h] = bf16_bits(t[h])
    return arr


def test_prefill_at_the_largest_supported_length(gpu_lib):
    w = PrefillWorkload("max_length", S=S_MAX, Hq=2, Hkv=1, d=128, n_ret=1,
                        window=4096, r=16, block=64, top_k=8, seed=11,
                        retrieval_heads=(1,))
    n_b = w.n_blocks
    assert n_b * 64 == S_MAX and n_b == 262143
    print(f"[max] prefill S={S_MAX}: drawing inputs", flush=True)
    x = make_prefill(w, device="cuda")
    pq = torch.from_numpy(x["p_q"]).cuda()
    pk = torch.from_numpy(x["p_k"]).cuda()
    out, lse, sel, cnt = gpu_lib.hybrid_attn_prefill(
        x["q"], x["k"], x["v"], x["is_retrieval"], w.window, pq, pk, w.top_k,
        r=w.r, want_lse=True, want_sel=True)
    torch.cuda.synchronize()
    print("[max] GPU run done; copying inputs to the host", flush=True)
    sel, cnt = sel.cpu().numpy()[0], cnt.cpu().numpy()[0]
    qbits = _host_heads(x["q"], [0, 1])
    kbits = bf16_bits(x["k"])
    vbits = bf16_bits(x["v"])

    rng = np.random.default_rng(5)
    rows = sorted({0, 1, 2, 3, n_b // 2 - 1, n_b // 2, n_b - 2, n_b - 1} |
                  set(int(i) for i in rng.integers(4, n_b - 2, 8)))
    ora = oracle.hybrid_prefill(qbits, kbits, kbits, x["is_retrieval"],
                                w.window, x["p_q"], x["p_k"], 64, w.top_k,
                                heads=[1], query_blocks=[], sel_rows=rows)
    fn = parity.prefill_rows_fn(x, qbits, kbits, 0, 1)
    ties = parity.compare_selection(
        sel[rows], cnt[rows], ora["sel"][0][rows], ora["sel_count"][0][rows],
        ora["kth"][0][rows], lambda i: fn(rows[i]),
        parity.prefill_required(lambda i: rows[i]), "max length")
    parity.assert_tie_rate(ties, len(rows), "max length")
    print(f"[max] {len(rows)} selection rows identical except {len(ties)} "
          "logged ties", flush=True)

    qbs = [0, 1, n_b // 2, n_b - 1]
    override = {0: {qb: sel[qb, :cnt[qb]] for qb in qbs}}
    ora = oracle.hybrid_prefill(qbits, kbits, vbits, x["is_retrieval"],
                                w.window, x["p_q"], x["p_k"], 64, w.top_k,
                                sel_override=override, heads=[0, 1],
                                query_blocks=qbs)
    worst = 0.0
    for h in (0, 1):
        for qb in qbs:
            s = slice(qb * 64, qb * 64 + 64)
            err = parity.max_abs(out[h, s].float().cpu().numpy(),
                                 ora["out"][h, s])
            assert err <= parity.OUT_TOL, (h, qb, err)
            worst = max(worst, err)
            parity.check_prefill_lse(lse[h:h + 1, s].cpu().numpy(),
                                     ora["lse"][h:h + 1, s],
                                     x["is_retrieval"][h:h + 1],
                                     f"max length h={h} qb={qb}")
    print(f"[max] outputs of {len(qbs)} query blocks x 2 heads: max |dO| "
          f"{worst:.2e}", flush=True)


def test_decode_after_the_largest_supported_prefill(gpu_lib):
    L = S_MAX + 1  # the prompt plus the new token (a one-token last block)
    print(f"[max] decode L={L}", flush=True)
    y = make_decode(_dec_wl(1, L, Hq=2, Hkv=1, ret=(1,), window=8192,
                            top_k=64, seed=13), device="cuda")
    dec_check(gpu_lib, y, "decode max length")
