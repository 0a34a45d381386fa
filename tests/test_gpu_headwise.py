"""GPU parity of rtp_headwise_prefill (through the C ABI) against the oracle:
a window per streaming head, retrieval heads sparse or full, and the block
centroids for decode as an epilogue."""
import numpy as np
import pytest
import torch

import oracle
from tests import parity
from workloads import PrefillWorkload, make_prefill, bf16_bits

pytestmark = pytest.mark.gpu


def _wl(S, Hq, Hkv, ret, top_k, seed=0):
    return PrefillWorkload("t", S=S, Hq=Hq, Hkv=Hkv, d=128, n_ret=len(ret),
                           window=64, r=16, block=64, top_k=top_k, seed=seed,
                           retrieval_heads=tuple(ret))


def _dev(x):
    return (x["q"].cuda(), x["k"].cuda(), x["v"].cuda(),
            torch.from_numpy(x["p_q"]).cuda(), torch.from_numpy(x["p_k"]).cuda())


def _bits(x):
    return bf16_bits(x["q"]), bf16_bits(x["k"]), bf16_bits(x["v"])


def test_sparse_mode_with_a_window_per_head(gpu_lib):
    # streaming heads of one KV group with different windows (1, 100, 700,
    # 8192 > S, and one shared by two heads); ragged S; selection as usual
    S = 64 * 20 + 23
    x = make_prefill(_wl(S, Hq=8, Hkv=2, ret=(1, 6), top_k=5))
    windows = [1, 0, 100, 700, 8192, 100, 0, 333]
    q, k, v, pq, pk = _dev(x)
    out, lse, sel, cnt, cent = gpu_lib.headwise_prefill(
        q, k, v, x["is_retrieval"], windows, pq, pk, 5, want_lse=True,
        want_sel=True, want_centroids=True)
    torch.cuda.synchronize()
    qb_, kb_, vb_ = _bits(x)
    gsel, gcnt = sel.cpu().numpy(), cnt.cpu().numpy()
    n_b = -(-S // 64)
    override = {rho: {qb: gsel[rho, qb, :gcnt[rho, qb]] for qb in range(n_b)}
                for rho in range(2)}
    ora = oracle.hybrid_prefill(qb_, kb_, vb_, x["is_retrieval"], windows,
                                x["p_q"], x["p_k"], 64, 5)
    for rho, h in enumerate((1, 6)):
        fn = parity.prefill_rows_fn(x, qb_, kb_, rho, h)
        parity.compare_selection(gsel[rho], gcnt[rho], ora["sel"][rho],
                                 ora["sel_count"][rho], ora["kth"][rho], fn,
                                 parity.prefill_required(int),
                                 f"headwise rho={rho}")
    ref = oracle.hybrid_prefill(qb_, kb_, vb_, x["is_retrieval"], windows,
                                x["p_q"], x["p_k"], 64, 5,
                                sel_override=override)
    assert parity.max_abs(parity.bf16_to_f32(out), ref["out"]) <= parity.OUT_TOL
    parity.check_prefill_lse(lse.cpu().numpy(), ref["lse"], x["is_retrieval"],
                             "headwise sparse")
    # window 1 returns V bitwise
    assert torch.equal(out[0].cpu(), x["v"][0])
    c = cent.cpu().numpy()
    assert np.abs(c - ora["centroids"]).max() <= 1e-5 * np.abs(ora["centroids"]).max()


@pytest.mark.parametrize("S", [64 * 40, 64 * 33 + 5])
def test_full_mode_matches_oracle_and_decode_centroids(gpu_lib, S):
    # retrieval heads attend every earlier key; the centroid epilogue equals
    # the decode-side centroid build of a cache that holds this sequence
    x = make_prefill(_wl(S, Hq=8, Hkv=2, ret=(0, 3, 5), top_k=4))
    windows = [0, 256, 64, 0, 1000, 0, 64, 128]
    q, k, v, pq, pk = _dev(x)
    out, lse, sel, cnt, cent = gpu_lib.headwise_prefill(
        q, k, v, x["is_retrieval"], windows, None, pk, 4, retrieval="full",
        want_lse=True, want_centroids=True)
    torch.cuda.synchronize()
    assert sel is None and cnt is None
    qb_, kb_, vb_ = _bits(x)
    ora = oracle.hybrid_prefill(qb_, kb_, vb_, x["is_retrieval"], windows,
                                x["p_q"], x["p_k"], 64, 4, retrieval_full=True)
    assert parity.max_abs(parity.bf16_to_f32(out), ora["out"]) <= parity.OUT_TOL
    lerr = parity.check_prefill_lse(lse.cpu().numpy(), ora["lse"],
                                    x["is_retrieval"], "headwise full",
                                    retrieval_full=True)
    print(f"[lse] headwise full S={S}: {lerr['window']:.2e}", flush=True)
    c = cent.cpu().numpy()
    assert np.abs(c - ora["centroids"]).max() <= 1e-5 * np.abs(ora["centroids"]).max()
    # decode cache [1, Hkv, Lmax, d] holding the sequence
    Lmax = -(-S // 64) * 64 + 64
    kc = torch.zeros((1, 2, Lmax, 128), dtype=torch.bfloat16, device="cuda")
    kc[0, :, :S] = k
    cl = torch.tensor([S], dtype=torch.int32, device="cuda")
    dec = gpu_lib.build_centroids(kc, cl, x["is_retrieval"], pk).cpu().numpy()
    n_full = S // 64
    ref = dec[0, :, :n_full]
    assert np.abs(c[:, :n_full] - ref).max() <= 1e-5 * np.abs(ref).max()


def test_equal_windows_match_the_single_window_entry_point(gpu_lib):
    S = 64 * 30 + 9
    x = make_prefill(_wl(S, Hq=4, Hkv=1, ret=(2,), top_k=6))
    q, k, v, pq, pk = _dev(x)
    a = gpu_lib.hybrid_attn_prefill(q, k, v, x["is_retrieval"], 200, pq, pk, 6)
    b = gpu_lib.headwise_prefill(q, k, v, x["is_retrieval"], [200] * 4, pq,
                                 pk, 6)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_full_prefill_then_sparse_decode_recipe(gpu_lib):
    # The deployment recipe end to end: prefill with full retrieval heads and
    # the key clustering as its epilogue; the sequence and its centroids
    # become a decode cache; one appended token completes a block (its
    # centroid added on the decode side); then a decode step runs the
    # retrieval heads sparse over those centroids. Checked against the
    # oracle's decode, which derives every centroid from the cache itself.
    S = 64 * 151 - 1
    ret = (1, 6)
    x = make_prefill(_wl(S, Hq=8, Hkv=2, ret=ret, top_k=8, seed=3))
    windows = [512] * 8
    q, k, v, pq, pk = _dev(x)
    _, _, _, _, cent = gpu_lib.headwise_prefill(
        q, k, v, x["is_retrieval"], windows, None, pk, 8, retrieval="full",
        want_centroids=True)
    Lmax = 64 * 160
    kc = torch.zeros((1, 2, Lmax, 128), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kc[0, :, :S] = k
    vc[0, :, :S] = v
    dcent = torch.zeros((1, 2, Lmax // 64, 16), dtype=torch.float32,
                        device="cuda")
    n_full = S // 64
    dcent[0, :, :n_full] = cent[:, :n_full]
    cl = torch.tensor([S], dtype=torch.int32, device="cuda")
    gen = torch.Generator().manual_seed(11)
    kn = torch.randn(1, 2, 128, generator=gen).to(torch.bfloat16).cuda()
    vn = torch.randn(1, 2, 128, generator=gen).to(torch.bfloat16).cuda()
    gpu_lib.decode_append(kc, vc, cl, kn, vn, x["is_retrieval"], pk, dcent)
    qd = torch.randn(1, 8, 128, generator=gen).to(torch.bfloat16)
    out, lse, sel = gpu_lib.hybrid_attn_decode(
        qd.cuda(), kc, vc, cl, x["is_retrieval"], 512, pq, dcent, 8,
        n_recent=2, want_lse=True, want_sel=True)
    torch.cuda.synchronize()
    assert int(cl.item()) == S + 1
    kcb, vcb = bf16_bits(kc.cpu()), bf16_bits(vc.cpu())
    ora = oracle.hybrid_decode(bf16_bits(qd), kcb, vcb, np.array([S + 1]),
                               x["is_retrieval"], 512, x["p_q"], x["p_k"], 64,
                               8, 2)
    g = sel.cpu().numpy()
    n_b = -(-(S + 1) // 64)
    override = {}
    for rho, h in enumerate(ret):
        c_o = ora["centroids"][(0, rho)]
        qt = x["p_q"][rho] @ oracle.bf16_to_f32(bf16_bits(qd[0, h]))
        gcnt = int((g[0, rho] >= 0).sum())
        ties = parity.compare_selection(
            g[0, rho][None], np.array([gcnt]), ora["sel"][0, rho][None],
            ora["sel_count"][0, rho][None], ora["kth"][0, rho][None],
            parity.decode_scores_fn(c_o, qt, n_b, 2),
            parity.decode_required(n_b, 2), f"recipe rho={rho}")
        if ties:
            override[(0, rho)] = g[0, rho][:gcnt]
    if override:  # attend under the GPU's own (equally valid) choice
        ora = oracle.hybrid_decode(bf16_bits(qd), kcb, vcb, np.array([S + 1]),
                                   x["is_retrieval"], 512, x["p_q"],
                                   x["p_k"], 64, 8, 2, sel_override=override)
    o_g = parity.bf16_to_f32(out)
    for h in range(8):
        assert parity.max_abs(o_g[0, h], ora["out"][0, h]) <= parity.OUT_TOL, h
        assert abs(lse.cpu().numpy()[0, h] - ora["lse"][0, h]) <= \
            parity.LSE_TOL_BF16_SUM
