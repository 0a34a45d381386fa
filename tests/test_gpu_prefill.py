"""GPU parity of hybrid prefill (through the C ABI) against the CPU oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
from tests import parity
from workloads import PrefillWorkload, TINY, make_prefill, bf16_bits

pytestmark = pytest.mark.gpu


def _wl(S, Hq, Hkv, ret, window, top_k, r=16, seed=0, needles=0, d=128):
    return PrefillWorkload("t", S=S, Hq=Hq, Hkv=Hkv, d=d, n_ret=len(ret),
                           window=window, r=r, block=64, top_k=top_k,
                           seed=seed, retrieval_heads=tuple(ret),
                           needles=needles)


def _to_dev(x):
    dev = dict(x)
    for key in ("q", "k", "v"):
        dev[key] = x[key].cuda()
    dev["p_q_t"] = torch.from_numpy(x["p_q"]).cuda()
    dev["p_k_t"] = torch.from_numpy(x["p_k"]).cuda()
    return dev


def _bits(x):
    return bf16_bits(x["q"]), bf16_bits(x["k"]), bf16_bits(x["v"])


def _run_gpu(rtp, d, **kw):
    out, lse, sel, cnt = rtp.hybrid_attn_prefill(
        d["q"], d["k"], d["v"], d["is_retrieval"], d["window"], d["p_q_t"],
        d["p_k_t"], d["top_k"], r=d["r"], want_lse=True, want_sel=True, **kw)
    torch.cuda.synchronize()
    return out, lse, sel, cnt


def full_check(rtp, x, label):
    """Whole-layer comparison: selection, outputs, LSE."""
    d = _to_dev(x)
    qb_, kb_, vb_ = _bits(x)
    out, lse, sel, cnt = _run_gpu(rtp, d)
    ora = oracle.hybrid_prefill(qb_, kb_, vb_, x["is_retrieval"], x["window"],
                                x["p_q"], x["p_k"], x["block"], x["top_k"])
    heads = list(x["retrieval_heads"])
    n_b = -(-x["q"].shape[1] // 64)
    gsel, gcnt = sel.cpu().numpy(), cnt.cpu().numpy()
    ties = []
    for rho, h in enumerate(heads):
        fn = parity.prefill_rows_fn(x, qb_, kb_, rho, h)
        ties += parity.compare_selection(gsel[rho], gcnt[rho], ora["sel"][rho],
                                         ora["sel_count"][rho], ora["kth"][rho],
                                         fn, parity.prefill_required(int),
                                         f"{label} rho={rho}")
    # attention under the GPU's own selection (equal to the oracle's except
    # at logged ties)
    override = {rho: {qb: gsel[rho, qb, :gcnt[rho, qb]] for qb in range(n_b)}
                for rho in range(len(heads))}
    ref = ora if not ties else oracle.hybrid_prefill(
        qb_, kb_, vb_, x["is_retrieval"], x["window"], x["p_q"], x["p_k"],
        x["block"], x["top_k"], sel_override=override)
    err = parity.max_abs(parity.bf16_to_f32(out), ref["out"])
    assert err <= parity.OUT_TOL, (label, err)
    lerr = parity.check_prefill_lse(lse.cpu().numpy(), ref["lse"],
                                    x["is_retrieval"], label)
    print(f"[lse] {label}: window {lerr['window']:.2e} sparse "
          f"{lerr['sparse']:.2e}", flush=True)
    assert not torch.isnan(out.float()).any()
    return dict(err=err, lse_err=max(lerr.values()), ties=ties, out=out,
                sel=gsel, cnt=gcnt, ora=ora)


def test_tiny_workload_full_parity(gpu_lib):
    x = make_prefill(TINY)
    r = full_check(gpu_lib, x, "tiny")
    print(f"tiny: max|dO|={r['err']:.2e} max|dLSE|={r['lse_err']:.2e} "
          f"ties={len(r['ties'])}")


@pytest.mark.parametrize("S", [1, 63, 64, 65, 130, 1000, 1111])
def test_ragged_lengths(gpu_lib, S):
    x = make_prefill(_wl(S, Hq=4, Hkv=2, ret=(1, 2), window=100, top_k=3,
                         seed=S))
    full_check(gpu_lib, x, f"S={S}")


@pytest.mark.parametrize("r", [32, 48, 64])
def test_indexer_ranks(gpu_lib, r):
    # other indexer ranks stage a different number of key blocks per step
    x = make_prefill(_wl(64 * 37 + 11, Hq=4, Hkv=1, ret=(0, 3), window=150,
                         top_k=5, r=r))
    full_check(gpu_lib, x, f"r{r}")


@pytest.mark.parametrize("Hq,Hkv,ret,S", [
    (40, 2, (0, 21, 39), 64 * 19 + 9),
    (128, 8, (0, 17, 64, 127), 64 * 5 + 1),
])
def test_wide_groups_and_the_head_limit(gpu_lib, Hq, Hkv, ret, S):
    # 20 heads per KV group (window-kernel work items then span query
    # blocks), and the largest head count the library takes (128, groups of
    # 16, retrieval heads at both ends)
    x = make_prefill(_wl(S, Hq=Hq, Hkv=Hkv, ret=ret, window=333, top_k=3,
                         seed=Hq))
    full_check(gpu_lib, x, f"Hq{Hq}")


def test_nothing_is_read_past_the_inputs(gpu_lib):
    # Q, K and V as the front of buffers whose remainder is NaN: a read past
    # any of them (the ragged last block of the last head) would reach the
    # output even with weight 0, so the results must equal those of plain
    # tensors bit for bit
    x = make_prefill(_wl(64 * 30 + 5, Hq=4, Hkv=2, ret=(1, 3), window=100,
                         top_k=3, seed=9))
    d = _to_dev(x)
    padded = dict(d)
    for key in ("q", "k", "v"):
        t = d[key]
        buf = torch.full((t.numel() + 64 * 128 * 8,), float("nan"),
                         dtype=t.dtype, device=t.device)
        padded[key] = buf[:t.numel()].view(t.shape)
        padded[key].copy_(t)
    a = _run_gpu(gpu_lib, d)
    b = _run_gpu(gpu_lib, padded)
    for u, v in zip(a, b):
        if u.dtype == torch.bfloat16:
            u, v = u.view(torch.int16), v.view(torch.int16)
        assert torch.equal(u, v)


def test_every_head_retrieval_one_head_per_group(gpu_lib):
    # G = 1 and no streaming heads: only the sparse kernel runs
    x = make_prefill(_wl(64 * 21 + 3, Hq=3, Hkv=3, ret=(0, 1, 2), window=64,
                         top_k=4))
    full_check(gpu_lib, x, "allret")


@pytest.mark.parametrize("window,top_k", [(1, 0), (64, 1), (65, 2),
                                          (4096, 100)])
def test_window_and_budget_edges(gpu_lib, window, top_k):
    # window 1 (self only), k = 0 (sink + diagonal), k >= n_b (everything)
    x = make_prefill(_wl(1536, Hq=8, Hkv=2, ret=(0, 5, 6), window=window,
                         top_k=top_k, seed=window))
    full_check(gpu_lib, x, f"w={window},k={top_k}")


def test_window_one_returns_v_bitwise(gpu_lib):
    x = make_prefill(_wl(700, Hq=4, Hkv=1, ret=(), window=1, top_k=1))
    d = _to_dev(x)
    out = gpu_lib.hybrid_attn_prefill(d["q"], d["k"], d["v"],
                                      d["is_retrieval"], 1, None, None, 1)
    torch.cuda.synchronize()
    for h in range(4):
        assert torch.equal(out[h].cpu(), x["v"][0])


def test_dense_kernel_equals_oracle_full_coverage(gpu_lib):
    S = 1200
    x = make_prefill(_wl(S, Hq=8, Hkv=2, ret=(), window=S, top_k=1, seed=5))
    d = _to_dev(x)
    out, lse = gpu_lib.dense_attn_prefill(d["q"], d["k"], d["v"],
                                          want_lse=True)
    torch.cuda.synchronize()
    ora = oracle.hybrid_prefill(*_bits(x), x["is_retrieval"], S, x["p_q"],
                                x["p_k"], 64, 1)
    assert parity.max_abs(parity.bf16_to_f32(out), ora["out"]) <= parity.OUT_TOL
    lerr = parity.check_prefill_lse(lse.cpu().numpy(), ora["lse"],
                                    x["is_retrieval"], "dense")
    print(f"[lse] dense: {lerr['window']:.2e}", flush=True)


def test_hybrid_with_full_budget_equals_dense(gpu_lib):
    # window >= S and k >= n_b - 2: hybrid prefill is dense causal attention
    S = 960
    x = make_prefill(_wl(S, Hq=8, Hkv=2, ret=(1, 4, 7), window=S, top_k=64,
                         seed=7))
    d = _to_dev(x)
    out = _run_gpu(gpu_lib, d)[0]
    dense = gpu_lib.dense_attn_prefill(d["q"], d["k"], d["v"])
    torch.cuda.synchronize()
    # The two kernels differ only in rounding (the window kernel sums the
    # fp32 weights, the sparse one their bf16-rounded copies), so they agree
    # to about one bf16 ulp of each output: allow two.
    a, b = out.float(), dense.float()
    tol = 2.0 ** -6 * b.abs().clamp_min(0.5)
    excess = ((a - b).abs() - tol).max().item()
    assert excess <= 0, excess


@pytest.mark.parametrize("with_diag", [True, False])
def test_selection_override_is_used(gpu_lib, with_diag):
    # an explicit selection skips the indexer; outputs follow it exactly,
    # also when a row leaves out its own diagonal block
    S = 640
    x = make_prefill(_wl(S, Hq=2, Hkv=1, ret=(0,), window=32, top_k=2))
    d = _to_dev(x)
    n_b = S // 64
    sel = np.full((1, n_b, 4), -1, dtype=np.int32)
    cnt = np.zeros((1, n_b), dtype=np.int32)
    override = {0: {}}
    for qb in range(n_b):
        keep = {0, qb} if with_diag or qb == 0 else {0}
        s = sorted(keep | ({qb // 2} if qb >= 2 else set()))
        sel[0, qb, :len(s)] = s
        cnt[0, qb] = len(s)
        override[0][qb] = np.array(s)
    out = gpu_lib.hybrid_attn_prefill(
        d["q"], d["k"], d["v"], x["is_retrieval"], 32, None, None, 2,
        sel=torch.from_numpy(sel).cuda(), sel_count=torch.from_numpy(cnt).cuda())
    torch.cuda.synchronize()
    ora = oracle.hybrid_prefill(*_bits(x), x["is_retrieval"], 32, x["p_q"],
                                x["p_k"], 64, 2, sel_override=override)
    assert parity.max_abs(parity.bf16_to_f32(out), ora["out"]) <= parity.OUT_TOL


def test_poisoned_keys_outside_the_sets_leave_output_unchanged(gpu_lib):
    # Keys no query of a 64-query tile can see are never read; values of
    # keys masked for some rows are multiplied by exactly 0. Poison K with NaN
    # and V with 1e4 outside the union of windows / selections of the last
    # query block; its outputs must stay bitwise equal.
    S, w = 1024, 100
    x = make_prefill(_wl(S, Hq=4, Hkv=1, ret=(2,), window=w, top_k=2))
    d = _to_dev(x)
    out0, _, sel, cnt = _run_gpu(gpu_lib, d)
    qb = S // 64 - 1
    keep = set(range(qb * 64 - w + 1, S))
    s = sel[0, qb, :cnt[0, qb]].cpu().numpy()
    for b in s:
        keep |= set(range(b * 64, b * 64 + 64))
    bad = torch.tensor(sorted(set(range(S)) - keep))
    k2, v2 = d["k"].clone(), d["v"].clone()
    k2[:, bad] = float("nan")
    v2[:, bad] = 1e4
    out1 = gpu_lib.hybrid_attn_prefill(
        d["q"], k2, v2, x["is_retrieval"], w, None, None, 2, sel=sel,
        sel_count=cnt)
    torch.cuda.synchronize()
    assert torch.equal(out1[:, qb * 64:], out0[:, qb * 64:])


def test_deterministic(gpu_lib):
    x = make_prefill(_wl(2048, Hq=8, Hkv=2, ret=(3,), window=300, top_k=5))
    d = _to_dev(x)
    a = _run_gpu(gpu_lib, d)
    b = _run_gpu(gpu_lib, d)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_identity_projection_selects_true_top_blocks(gpu_lib):
    # r = d = 128 with P = I: scores are block-averaged true logits; the GPU
    # indexer must pick the oracle's exact top blocks (up to logged ties).
    S = 2048
    x = make_prefill(_wl(S, Hq=2, Hkv=1, ret=(0, 1), window=64, top_k=6,
                         r=128))
    eye = np.broadcast_to(np.eye(128, dtype=np.float32), (2, 128, 128)).copy()
    x["p_q"], x["p_k"] = eye, eye
    x["r"] = 128
    full_check(gpu_lib, x, "identity")


@pytest.mark.parametrize("S,top_k", [(4096, 9), (64 * 700, 300)])
def test_indexer_select_kth_scores_and_centroids(gpu_lib, S, top_k):
    # a small and a large budget; both report the k-th and (k+1)-th scores
    x = make_prefill(_wl(S, Hq=8, Hkv=2, ret=(0, 3, 6), window=64,
                         top_k=top_k, seed=11))
    d = _to_dev(x)
    sel, cnt, kth, cent = gpu_lib.indexer_select(
        d["q"], d["k"], x["is_retrieval"], d["p_q_t"], d["p_k_t"], top_k,
        kth=True, centroids=True)
    torch.cuda.synchronize()
    ora_sel = oracle.hybrid_prefill(*_bits(x), x["is_retrieval"], 64,
                                    x["p_q"], x["p_k"], 64, top_k,
                                    heads=[0, 3, 6], query_blocks=[0],
                                    sel_rows=range(S // 64))
    for rho, h in enumerate((0, 3, 6)):
        fn = parity.prefill_rows_fn(x, *_bits(x)[:2], rho, h)
        parity.compare_selection(sel.cpu().numpy()[rho], cnt.cpu().numpy()[rho],
                                 ora_sel["sel"][rho], ora_sel["sel_count"][rho],
                                 ora_sel["kth"][rho], fn,
                                 parity.prefill_required(int), f"kth rho={rho}")
    k_g, k_o = kth.cpu().numpy(), ora_sel["kth"]
    both = ~np.isnan(k_o)
    assert np.array_equal(np.isnan(k_g), np.isnan(k_o))
    rel = np.abs(k_g[both] - k_o[both]) / np.maximum(np.abs(k_o[both]), 1e-3)
    assert rel.max() < 1e-4, rel.max()
    c_g, c_o = cent.cpu().numpy(), ora_sel["centroids"]
    assert np.abs(c_g - c_o).max() <= 1e-5 * np.abs(c_o).max() + 1e-6


def test_reference_restart_when_an_early_key_dominates(gpu_lib):
    # Every query equals u and key 0 is 60 u/|u|: its score exceeds the
    # diagonal block's scores by far more than the kernels' no-rescale range,
    # so window and retrieval heads must restart with a raised reference and
    # still match the exact softmax.
    S = 512
    x = make_prefill(_wl(S, Hq=4, Hkv=1, ret=(1, 3), window=S, top_k=2))
    g = torch.Generator().manual_seed(7)
    u = torch.randn(128, generator=g)
    q = u.to(torch.bfloat16).expand(4, S, 128).contiguous()
    k = x["k"].clone()
    k[0, 0] = (60.0 * u / u.norm()).to(torch.bfloat16)
    x["q"], x["k"] = q, k
    r = full_check(gpu_lib, x, "restart")
    assert np.isfinite(r["out"].float().cpu().numpy()).all()


def test_indexer_equal_scores_keep_the_lowest_blocks(gpu_lib):
    # Every key equal => every candidate block of a row scores the same, so
    # the kept set is fixed by the tie rule alone: blocks 1..k (lower index
    # first), plus the sink and the diagonal. Rows longer than 2048
    # candidates put more keys in the threshold's value bin than the
    # selection gathers in LDS, which exercises its in-place search.
    S, k = 2200 * 64, 37
    x = make_prefill(_wl(S, Hq=2, Hkv=1, ret=(1,), window=64, top_k=k))
    kc = torch.full_like(x["k"], 0.5)
    d = _to_dev(dict(x, k=kc))
    sel, cnt, kth, _ = gpu_lib.indexer_select(
        d["q"], d["k"], x["is_retrieval"], d["p_q_t"], d["p_k_t"], k, kth=True)
    torch.cuda.synchronize()
    sel, cnt, kth = sel.cpu().numpy()[0], cnt.cpu().numpy()[0], kth.cpu().numpy()[0]
    n_b = S // 64
    for qb in range(n_b):
        cand = list(range(1, qb))[:k]
        want = sorted({0, qb} | set(cand))
        assert int(cnt[qb]) == len(want), qb
        assert list(sel[qb][:cnt[qb]]) == want, qb
        if qb - 1 > k:  # s_k and s_{k+1} both exist and are equal
            assert kth[qb][0] == kth[qb][1], qb
