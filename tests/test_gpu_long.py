"""GPU parity of the selections on very long rows (through the C ABI).

Prefill rows past 16 384 and past 32 768 candidate blocks (over a million
and over two million tokens), checked against the oracle on a stratified
sample of rows, and a layer whose scores are all equal, where the kept set
is known by construction (the tie rule alone decides it). Decode block
choices past 16 384 candidates, on both selection paths (per-wave for
budgets up to 64, block-wide above), and a cache of over 32 768 candidate
blocks whose centroid scores are all equal.
"""
import numpy as np
import pytest
import torch

import oracle
from tests import parity
from tests.test_gpu_decode import _wl as _dec_wl, check as dec_check
from workloads import PrefillWorkload, make_prefill, make_decode, bf16_bits

pytestmark = pytest.mark.gpu


def _pwl(S, Hq, Hkv, ret, top_k, seed=0):
    return PrefillWorkload("long", S=S, Hq=Hq, Hkv=Hkv, d=128, n_ret=len(ret),
                           window=64, r=16, block=64, top_k=top_k, seed=seed,
                           retrieval_heads=tuple(ret))


def _rows(n_b, seed, stride=64):
    rng = np.random.default_rng(seed)
    rows = {0, 1, 2, 3, n_b // 2, n_b - 2, n_b - 1}
    for lo in range(0, n_b, stride):
        rows.add(int(rng.integers(lo, min(n_b, lo + stride))))
    return sorted(rows)


def test_prefill_rows_past_16k_candidates(gpu_lib):
    # 17 000 blocks and a ragged tail: the last rows hold ~17 000 candidates
    S = 64 * 17000 + 21
    w = _pwl(S, Hq=2, Hkv=1, ret=(1,), top_k=8, seed=5)
    print(f"[long] prefill S={S}", flush=True)
    x = make_prefill(w, device="cuda")
    pq = torch.from_numpy(x["p_q"]).cuda()
    pk = torch.from_numpy(x["p_k"]).cuda()
    sel, cnt, kth, _ = gpu_lib.indexer_select(x["q"], x["k"], x["is_retrieval"],
                                              pq, pk, w.top_k, kth=True)
    torch.cuda.synchronize()
    n_b = w.n_blocks
    rows = _rows(n_b, 7, stride=64)
    qbits = np.empty((2, S, 128), np.uint16)
    qbits[1] = bf16_bits(x["q"][1])
    kbits = bf16_bits(x["k"])
    ora = oracle.hybrid_prefill(qbits, kbits, kbits, x["is_retrieval"], 64,
                                x["p_q"], x["p_k"], 64, w.top_k, heads=[1],
                                query_blocks=[], sel_rows=rows)
    g_sel, g_cnt = sel.cpu().numpy()[0], cnt.cpu().numpy()[0]
    fn = parity.prefill_rows_fn(x, qbits, kbits, 0, 1)
    ties = parity.compare_selection(
        g_sel[rows], g_cnt[rows], ora["sel"][0][rows], ora["sel_count"][0][rows],
        ora["kth"][0][rows], lambda i: fn(rows[i]),
        parity.prefill_required(lambda i: rows[i]), "past16k")
    parity.assert_tie_rate(ties, len(rows), "past16k")
    k_g, k_o = kth.cpu().numpy()[0][rows], ora["kth"][0][rows]
    assert np.array_equal(np.isnan(k_g), np.isnan(k_o))
    both = ~np.isnan(k_o)
    rel = np.abs(k_g[both] - k_o[both]) / np.maximum(np.abs(k_o[both]), 1e-3)
    assert rel.max() < 1e-4, rel.max()
    print(f"[long] prefill past 16K: {len(rows)} rows, {len(ties)} ties",
          flush=True)


@pytest.mark.parametrize("top_k", [0, 1, 300, 600, 5000])
def test_prefill_streaming_select_budgets(gpu_lib, top_k):
    # Sequences past 4096 blocks take the fused scoring-and-selection
    # kernel. Budgets: none (sink and diagonal only), one, a few hundred
    # (buffers shrunk in registers), 600 (buffers too large for registers,
    # shrunk in memory), and more than any row has candidates (every block).
    S = 64 * 4200 + 13
    w = _pwl(S, Hq=2, Hkv=1, ret=(0,), top_k=top_k, seed=top_k)
    print(f"[long] streaming select S={S} top_k={top_k}", flush=True)
    x = make_prefill(w, device="cuda")
    pq = torch.from_numpy(x["p_q"]).cuda()
    pk = torch.from_numpy(x["p_k"]).cuda()
    sel, cnt, kth, _ = gpu_lib.indexer_select(x["q"], x["k"], x["is_retrieval"],
                                              pq, pk, top_k, kth=True)
    torch.cuda.synchronize()
    n_b = w.n_blocks
    rows = _rows(n_b, 11 + top_k, stride=32)
    qbits = np.empty((2, S, 128), np.uint16)
    qbits[0] = bf16_bits(x["q"][0])
    kbits = bf16_bits(x["k"])
    ora = oracle.hybrid_prefill(qbits, kbits, kbits, x["is_retrieval"], 64,
                                x["p_q"], x["p_k"], 64, top_k, heads=[0],
                                query_blocks=[], sel_rows=rows)
    g_sel, g_cnt = sel.cpu().numpy()[0], cnt.cpu().numpy()[0]
    fn = parity.prefill_rows_fn(x, qbits, kbits, 0, 0)
    ties = parity.compare_selection(
        g_sel[rows], g_cnt[rows], ora["sel"][0][rows], ora["sel_count"][0][rows],
        ora["kth"][0][rows], lambda i: fn(rows[i]),
        parity.prefill_required(lambda i: rows[i]), f"stream k={top_k}")
    parity.assert_tie_rate(ties, len(rows), f"stream k={top_k}")
    k_g, k_o = kth.cpu().numpy()[0][rows], ora["kth"][0][rows]
    assert np.array_equal(np.isnan(k_g), np.isnan(k_o))
    both = ~np.isnan(k_o)
    if both.any():
        rel = np.abs(k_g[both] - k_o[both]) / np.maximum(np.abs(k_o[both]), 1e-3)
        assert rel.max() < 1e-4, rel.max()


def test_prefill_equal_scores_past_32k_candidates(gpu_lib):
    # A zero query head: every block mean is 0, so every candidate scores 0
    # and the kept set is fixed by the tie rule alone (blocks 1..k, lowest
    # first, plus the sink and the diagonal); rows reach 33 000 candidates,
    # all equal, and s_k = s_{k+1} = 0.
    S = 64 * 33003 + 9
    k = 37
    w = _pwl(S, Hq=1, Hkv=1, ret=(0,), top_k=k, seed=9)
    print(f"[long] prefill equal scores S={S}", flush=True)
    x = make_prefill(w, device="cuda")
    x["q"].zero_()
    pq = torch.from_numpy(x["p_q"]).cuda()
    pk = torch.from_numpy(x["p_k"]).cuda()
    sel, cnt, kth, _ = gpu_lib.indexer_select(x["q"], x["k"], x["is_retrieval"],
                                              pq, pk, k, kth=True)
    torch.cuda.synchronize()
    sel, cnt, kth = sel.cpu().numpy()[0], cnt.cpu().numpy()[0], kth.cpu().numpy()[0]
    n_b = w.n_blocks
    qb = np.arange(n_b)
    long_rows = qb - 1 > k
    want = np.full((n_b, k + 2), -1, np.int64)
    want[long_rows, 0] = 0
    want[long_rows, 1:k + 1] = np.arange(1, k + 1)
    want[long_rows, k + 1] = qb[long_rows]
    for q in qb[~long_rows]:
        want[q, :q + 1] = np.arange(q + 1)
    assert np.array_equal(cnt, np.where(long_rows, k + 2, qb + 1))
    assert np.array_equal(sel, want)
    assert (kth[long_rows] == 0).all()


@pytest.mark.parametrize("top_k", [64, 65])
def test_decode_past_16k_candidates(gpu_lib, top_k):
    L = 64 * 17000 + 5
    print(f"[long] decode L={L} top_k={top_k}", flush=True)
    y = make_decode(_dec_wl(1, L, Hq=4, Hkv=1, ret=(1,), window=300,
                            top_k=top_k, seed=3))
    dec_check(gpu_lib, y, f"decode past16k k={top_k}")


def test_decode_equal_scores_past_32k_candidates(gpu_lib):
    # constant keys: every centroid, hence every candidate score, is equal;
    # 33 000 candidates take the block-wide select's two-scan path
    L = 64 * 33004 + 1
    top_k = 65
    print(f"[long] decode equal scores L={L}", flush=True)
    y = make_decode(_dec_wl(1, L, Hq=2, Hkv=1, ret=(0,), window=64,
                            top_k=top_k, seed=2), device="cuda")
    y["k_cache"].fill_(-0.25)
    dev = "cuda"
    cl = torch.from_numpy(y["cache_len"]).to(dev)
    pk = torch.from_numpy(y["p_k"]).to(dev)
    pq = torch.from_numpy(y["p_q"]).to(dev)
    cent = gpu_lib.build_centroids(y["k_cache"], cl, y["is_retrieval"], pk)
    _, _, sel = gpu_lib.hybrid_attn_decode(
        y["q"], y["k_cache"], y["v_cache"], cl, y["is_retrieval"], y["window"],
        pq, cent, top_k, n_recent=2, want_sel=True)
    torch.cuda.synchronize()
    n_b = -(-L // 64)
    got = [int(v) for v in sel.cpu().numpy()[0, 0] if v >= 0]
    assert got == [0] + list(range(1, top_k + 1)) + [n_b - 2, n_b - 1], \
        (got[:4], got[-4:])


@pytest.mark.parametrize("r", [32, 48, 128])
def test_prefill_streaming_select_other_ranks(gpu_lib, r):
    # the fused scoring-and-selection kernel for every operand width it is
    # built for beyond r = 16 (two key-block groups per load for r = 32, one
    # for wider), on a sequence just past 4096 blocks
    S = 64 * 4100 + 29
    w = PrefillWorkload("long", S=S, Hq=2, Hkv=1, d=128, n_ret=1, window=64,
                        r=r, block=64, top_k=40, seed=r,
                        retrieval_heads=(1,))
    print(f"[long] streaming select r={r} S={S}", flush=True)
    x = make_prefill(w, device="cuda")
    pq = torch.from_numpy(x["p_q"]).cuda()
    pk = torch.from_numpy(x["p_k"]).cuda()
    sel, cnt, kth, _ = gpu_lib.indexer_select(x["q"], x["k"], x["is_retrieval"],
                                              pq, pk, w.top_k, r=r, kth=True)
    torch.cuda.synchronize()
    n_b = w.n_blocks
    rows = _rows(n_b, 100 + r, stride=48)
    qbits = np.empty((2, S, 128), np.uint16)
    qbits[1] = bf16_bits(x["q"][1])
    kbits = bf16_bits(x["k"])
    ora = oracle.hybrid_prefill(qbits, kbits, kbits, x["is_retrieval"], 64,
                                x["p_q"], x["p_k"], 64, w.top_k, heads=[1],
                                query_blocks=[], sel_rows=rows)
    g_sel, g_cnt = sel.cpu().numpy()[0], cnt.cpu().numpy()[0]
    fn = parity.prefill_rows_fn(x, qbits, kbits, 0, 1)
    ties = parity.compare_selection(
        g_sel[rows], g_cnt[rows], ora["sel"][0][rows], ora["sel_count"][0][rows],
        ora["kth"][0][rows], lambda i: fn(rows[i]),
        parity.prefill_required(lambda i: rows[i]), f"stream r={r}")
    parity.assert_tie_rate(ties, len(rows), f"stream r={r}")
