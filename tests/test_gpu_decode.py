"""GPU parity of hybrid decode (through the C ABI) against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
from tests import parity
from workloads import DecodeWorkload, make_decode, bf16_bits

pytestmark = pytest.mark.gpu


def _wl(batch, L, Hq, Hkv, ret, window, top_k, n_recent=2, seed=0):
    return DecodeWorkload("t", batch=batch, L=L, Hq=Hq, Hkv=Hkv, d=128,
                          n_ret=len(ret), window=window, r=16, block=64,
                          top_k=top_k, n_recent=n_recent, seed=seed,
                          retrieval_heads=tuple(ret))


def run_gpu(rtp, y):
    dev = "cuda"
    kc, vc = y["k_cache"].to(dev), y["v_cache"].to(dev)
    cl = torch.from_numpy(y["cache_len"]).to(dev)
    pk = torch.from_numpy(y["p_k"]).to(dev)
    pq = torch.from_numpy(y["p_q"]).to(dev)
    cent = rtp.build_centroids(kc, cl, y["is_retrieval"], pk)
    out, lse, sel = rtp.hybrid_attn_decode(
        y["q"].to(dev), kc, vc, cl, y["is_retrieval"], y["window"], pq, cent,
        y["top_k"], n_recent=y["n_recent"], want_lse=True, want_sel=True)
    torch.cuda.synchronize()
    return out, lse, sel, cent


def check(rtp, y, label, seqs=None):
    out, lse, sel, cent = run_gpu(rtp, y)
    args = (bf16_bits(y["q"]), bf16_bits(y["k_cache"]),
            bf16_bits(y["v_cache"]), y["cache_len"], y["is_retrieval"],
            y["window"], y["p_q"], y["p_k"], 64, y["top_k"], y["n_recent"])
    ora = oracle.hybrid_decode(*args, seqs=seqs)
    seqs = range(len(y["cache_len"])) if seqs is None else seqs
    gsel = sel.cpu().numpy()
    gcent = cent.cpu().numpy()
    ties, override = [], {}
    for b in seqs:
        L = int(y["cache_len"][b])
        n_full, n_b = L // 64, -(-L // 64)
        for rho in range(len(y["retrieval_heads"])):
            c_o = ora["centroids"][(b, rho)]
            c_g = gcent[b, rho, :n_full]
            if n_full:
                assert np.abs(c_g - c_o).max() <= 1e-5 * max(
                    np.abs(c_o).max(), 1.0), (label, b, rho)
            g = gsel[b, rho]
            gcnt = int((g >= 0).sum())
            qt = (y["p_q"][rho] @ oracle.bf16_to_f32(bf16_bits(
                y["q"][b, y["retrieval_heads"][rho]])))
            t = parity.compare_selection(
                g[None], np.array([gcnt]), ora["sel"][b, rho][None],
                ora["sel_count"][b, rho][None], ora["kth"][b, rho][None],
                parity.decode_scores_fn(c_o, qt, n_b, y["n_recent"]),
                parity.decode_required(n_b, y["n_recent"]),
                f"{label} b={b} rho={rho}")
            if t:
                override[(b, rho)] = g[:gcnt]
            ties += t
    parity.assert_tie_rate(ties, len(list(seqs)) * len(y["retrieval_heads"]),
                           label)
    # rows whose choice differs at a logged near-tie are compared under the
    # GPU's own (equally valid) choice
    if override:
        ora = oracle.hybrid_decode(*args, seqs=seqs, sel_override=override)
    o_g = parity.bf16_to_f32(out)
    l_g = lse.cpu().numpy()
    worst = 0.0
    for b in seqs:
        for h in range(o_g.shape[1]):
            err = parity.max_abs(o_g[b, h], ora["out"][b, h])
            assert err <= parity.OUT_TOL, (label, b, h, err)
            lerr = abs(l_g[b, h] - ora["lse"][b, h])
            assert lerr <= parity.LSE_TOL_BF16_SUM, (label, b, h, lerr)
            worst = max(worst, lerr)
    print(f"[lse] decode {label}: {worst:.2e}, ties {len(ties)}", flush=True)
    return out, ora


def test_decode_ragged_batch(gpu_lib):
    y = make_decode(_wl(5, 6000, Hq=8, Hkv=2, ret=(1, 6), window=512,
                        top_k=8), cache_len=[6000, 4096, 777, 65, 4161])
    check(gpu_lib, y, "ragged")


@pytest.mark.parametrize("top_k", [0, 1, 37, 64, 65])
def test_decode_budgets_across_selection_paths(gpu_lib, top_k):
    # budgets up to 64 use the per-wave selection, larger ones the block-wide
    # radix select; 0 keeps only the sink and the recent blocks. The caches
    # hold 300-odd candidates, ragged, so the four quarters differ in size.
    y = make_decode(_wl(3, 64 * 300 + 17, Hq=8, Hkv=2, ret=(0, 5), window=256,
                        top_k=top_k), cache_len=[64 * 300 + 17, 64 * 71, 64 * 67 + 1])
    check(gpu_lib, y, f"budget{top_k}")


def test_decode_short_caches_keep_every_block(gpu_lib):
    y = make_decode(_wl(4, 200, Hq=4, Hkv=1, ret=(0, 2), window=64, top_k=8),
                    cache_len=[1, 63, 64, 130])
    out, ora = check(gpu_lib, y, "short")


def test_decode_full_coverage_equals_dense(gpu_lib):
    # window >= L and top_k >= n_b: every head attends the whole cache
    y = make_decode(_wl(3, 3000, Hq=8, Hkv=2, ret=(0, 3, 5), window=10 ** 6,
                        top_k=64), cache_len=[3000, 2049, 100])
    check(gpu_lib, y, "full")


def test_decode_window_one_returns_last_value(gpu_lib):
    y = make_decode(_wl(3, 500, Hq=4, Hkv=1, ret=(), window=1, top_k=1),
                    cache_len=[500, 1, 77])
    out = run_gpu(gpu_lib, y)[0].cpu()
    for b, L in enumerate([500, 1, 77]):
        for h in range(4):
            assert torch.equal(out[b, h], y["v_cache"][b, 0, L - 1])


@pytest.mark.parametrize("Hq", [16, 40])
def test_decode_many_heads_per_group(gpu_lib, Hq):
    # one KV head for all heads: 15 window heads share one pass over the
    # window; 39 need two (32 + 7)
    y = make_decode(_wl(2, 3000, Hq=Hq, Hkv=1, ret=(3,), window=700,
                        top_k=4), cache_len=[3000, 1800])
    check(gpu_lib, y, f"gqa{Hq}")


def test_cache_rows_past_each_length_are_never_read(gpu_lib):
    # NaN in every K/V row at or past a sequence's length: a row read there
    # would reach the output even with weight 0 (0 x NaN), so the outputs
    # must equal those of the clean cache bit for bit, in the block and the
    # clustered decode
    rtp = gpu_lib
    lens = [64 * 40 + 17, 64 * 9, 5, 64 * 63 + 63]
    y = make_decode(_wl(4, 64 * 64, Hq=8, Hkv=2, ret=(2, 5), window=200,
                        top_k=6), cache_len=lens)
    dev = "cuda"
    kc, vc = y["k_cache"].to(dev), y["v_cache"].to(dev)
    kn, vn = kc.clone(), vc.clone()
    for b, L in enumerate(lens):
        kn[b, :, L:] = float("nan")
        vn[b, :, L:] = float("nan")
    cl = torch.from_numpy(y["cache_len"]).to(dev)
    pk = torch.from_numpy(y["p_k"]).to(dev)
    pq = torch.from_numpy(y["p_q"]).to(dev)
    q = y["q"].to(dev)
    outs = []
    for k_, v_ in ((kc, vc), (kn, vn)):
        cent = rtp.build_centroids(k_, cl, y["is_retrieval"], pk)
        o1, l1, s1 = rtp.hybrid_attn_decode(
            q, k_, v_, cl, y["is_retrieval"], y["window"], pq, cent,
            y["top_k"], want_lse=True, want_sel=True)
        t = rtp.cluster_keys(k_, cl, y["is_retrieval"], pk, cent, iters=2)
        o2, l2, s2 = rtp.hybrid_attn_decode_clustered(
            q, k_, v_, cl, y["is_retrieval"], y["window"], pq, cent, t,
            y["top_k"], want_lse=True, want_sel=True)
        torch.cuda.synchronize()
        outs.append((o1, l1, s1, o2, l2, s2))
    for a, b in zip(*outs):
        if a.dtype == torch.bfloat16:
            a, b = a.view(torch.int16), b.view(torch.int16)
        assert torch.equal(a, b)
    assert not torch.isnan(outs[1][0].float()).any()
    assert not torch.isnan(outs[1][3].float()).any()


def test_decode_at_the_head_limit(gpu_lib):
    # 128 query heads over 2 KV heads: each group's 62 or 63 streaming heads
    # take two units, and the retrieval heads sit far apart
    y = make_decode(_wl(2, 1500, Hq=128, Hkv=2, ret=(5, 100), window=300,
                        top_k=6), cache_len=[1500, 1000])
    check(gpu_lib, y, "heads128")


def test_decode_runs_after_earlier_work_on_the_callers_stream(gpu_lib):
    # Streaming heads run on a stream of the library's own; they must still
    # see what the caller's stream wrote just before the call. V = 1 is made
    # by a kernel on a side stream right before decoding on that stream, so
    # every output is exactly 1 only if the whole step waited for it.
    y = make_decode(_wl(4, 20000, Hq=8, Hkv=2, ret=(1, 6), window=4096,
                        top_k=16), cache_len=[20000, 15000, 9000, 4097])
    dev = "cuda"
    kc = y["k_cache"].to(dev)
    cl = torch.from_numpy(y["cache_len"]).to(dev)
    pk = torch.from_numpy(y["p_k"]).to(dev)
    pq = torch.from_numpy(y["p_q"]).to(dev)
    cent = gpu_lib.build_centroids(kc, cl, y["is_retrieval"], pk)
    q = y["q"].to(dev)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        for _ in range(3):
            v1 = torch.empty_like(kc)
            v1.copy_(kc).mul_(0).add_(1)
            out = gpu_lib.hybrid_attn_decode(
                q, kc, v1, cl, y["is_retrieval"], y["window"], pq, cent,
                y["top_k"], n_recent=y["n_recent"])
            ones = bool((out == 1).all().item())
            assert ones, out.float().sub(1).abs().max().item()


def test_decode_deterministic(gpu_lib):
    y = make_decode(_wl(4, 4000, Hq=8, Hkv=2, ret=(2, 7), window=300,
                        top_k=6), cache_len=[4000, 3000, 2000, 999])
    a = run_gpu(gpu_lib, y)
    b = run_gpu(gpu_lib, y)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_decode_equal_centroid_scores_keep_the_lowest_blocks(gpu_lib):
    # constant keys => equal centroids => the kept blocks are the sink, the
    # lowest-index top_k candidates and the recent blocks; 4093 candidates
    # per row also exceed the selection's LDS gather size
    y = make_decode(_wl(2, 1 << 18, Hq=4, Hkv=1, ret=(2,), window=64,
                        top_k=64))
    y["k_cache"] = torch.full_like(y["k_cache"], -0.25)
    out, lse, sel, cent = run_gpu(gpu_lib, y)
    sel = sel.cpu().numpy()
    for b in range(2):
        n_b = int(y["cache_len"][b]) // 64
        want = [0] + list(range(1, 65)) + [n_b - 2, n_b - 1]
        got = [int(v) for v in sel[b, 0] if v >= 0]
        assert got == want, (b, got[:5], got[-5:])


def test_decode_append_matches_rebuild_and_oracle(gpu_lib):
    # Ragged caches, two of them one token short of a full block and one
    # already full. After an append the new rows sit at the old lengths,
    # cache_len grows by one (the full cache is left unchanged), the blocks
    # the token completed get centroids bitwise equal to a full rebuild, and
    # a decode step on the grown cache matches the oracle.
    Lmax = 64 * 40
    lens = [63, 64 * 7 + 63, 100, 64 * 12, Lmax]
    y = make_decode(_wl(len(lens), Lmax, Hq=8, Hkv=2, ret=(1, 6), window=200,
                        top_k=5), cache_len=lens, Lmax=Lmax)
    dev = "cuda"
    kc, vc = y["k_cache"].to(dev), y["v_cache"].to(dev)
    cl = torch.tensor(lens, dtype=torch.int32, device=dev)
    pk = torch.from_numpy(y["p_k"]).to(dev)
    cent = gpu_lib.build_centroids(kc, cl, y["is_retrieval"], pk)
    gen = torch.Generator().manual_seed(5)
    kn = torch.randn(len(lens), 2, 128, generator=gen).to(torch.bfloat16).to(dev)
    vn = torch.randn(len(lens), 2, 128, generator=gen).to(torch.bfloat16).to(dev)
    k_before = kc.clone()
    gpu_lib.decode_append(kc, vc, cl, kn, vn, y["is_retrieval"], pk, cent)
    torch.cuda.synchronize()
    grown = [L + 1 if L < Lmax else L for L in lens]
    assert cl.cpu().tolist() == grown
    for b, L in enumerate(lens):
        if L < Lmax:
            assert torch.equal(kc[b, :, L], kn[b]) and torch.equal(vc[b, :, L], vn[b])
        else:
            assert torch.equal(kc[b], k_before[b])
    rebuilt = gpu_lib.build_centroids(kc, cl, y["is_retrieval"], pk)
    torch.cuda.synchronize()
    assert torch.equal(cent, rebuilt)
    y2 = dict(y, k_cache=kc.cpu(), v_cache=vc.cpu(),
              cache_len=np.array(grown, dtype=np.int32))
    check(gpu_lib, y2, "after append")
