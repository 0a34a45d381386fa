"""GPU parity of the semantic K-cache clustering and of the clustered decode
step (through the C ABI) against the CPU oracle (oracle/cluster.py).

Each Lloyd step of the GPU is checked against the oracle's step taken from
the same starting centroids (the GPU's own): every token's cluster, except
near-ties (two centroids whose scores x.mu - |mu|^2/2 are within the bf16
split-product error of each other), each centroid as the mean of its
members, and the tables (every clustered token exactly once, ascending
within its cluster). The decode step is checked given the GPU's clusters:
the kept ids (empty clusters aside) up to near-ties at the cut, and the
output under the GPU's choice.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.cluster as oc
from tests import parity
from workloads import DecodeWorkload, make_decode, bf16_bits

pytestmark = pytest.mark.gpu

F64 = np.float64
# assignment near-tie band, relative to the magnitude of the two scores'
# terms: the GPU's products carry about 2^-16 of |x| |mu|
ASSIGN_BAND = 1e-4
# centroid tolerance (fp32 projections on both sides, means in fp64)
CENT_TOL = 2e-5


def _wl(batch, L, Hq, Hkv, ret, window, top_k, r=16, seed=0):
    return DecodeWorkload("t", batch=batch, L=L, Hq=Hq, Hkv=Hkv, d=128,
                          n_ret=len(ret), window=window, r=r, block=64,
                          top_k=top_k, n_recent=2, seed=seed,
                          retrieval_heads=tuple(ret))


class Gpu:
    def __init__(self, rtp, y, r=16):
        dev = "cuda"
        self.rtp, self.y, self.r = rtp, y, r
        self.kc, self.vc = y["k_cache"].to(dev), y["v_cache"].to(dev)
        self.q = y["q"].to(dev)
        self.cl = torch.from_numpy(y["cache_len"]).to(dev)
        self.pk = torch.from_numpy(y["p_k"]).to(dev)
        self.pq = torch.from_numpy(y["p_q"]).to(dev)
        self.cent = rtp.build_centroids(self.kc, self.cl, y["is_retrieval"],
                                        self.pk, r=r)
        self.tables = None

    def cluster(self, iters):
        self.tables = self.rtp.cluster_keys(
            self.kc, self.cl, self.y["is_retrieval"], self.pk, self.cent,
            iters=iters, n_recent=self.y["n_recent"], r=self.r,
            tables=self.tables)
        torch.cuda.synchronize()
        return self.read()

    def read(self):
        m, off, mem = (t.cpu().numpy() for t in self.tables)
        return m, off, mem, self.cent.cpu().numpy()

    def decode(self):
        out, lse, sel = self.rtp.hybrid_attn_decode_clustered(
            self.q, self.kc, self.vc, self.cl, self.y["is_retrieval"],
            self.y["window"], self.pq, self.cent, self.tables,
            self.y["top_k"], n_recent=self.y["n_recent"], r=self.r,
            want_lse=True, want_sel=True)
        torch.cuda.synchronize()
        return out, lse, sel


def _x(y, b, rho, m):
    """Oracle projected keys of the clustered tokens (fp64)."""
    g = y["retrieval_heads"][rho] // (y["q"].shape[1] // y["k_cache"].shape[1])
    k = oracle.bf16_to_f32(bf16_bits(y["k_cache"][b, g, 64:64 * m]))
    return oc.project_keys64(k, y["p_k"][rho])


def check_tables(m, off, mem, label):
    """Offsets consistent, every clustered token exactly once, members
    ascending within each cluster. Returns the assignment (cluster id per
    token 64 .. 64m-1)."""
    n_tok = 64 * (m - 1)
    assert off[0] == 0 and off[1] == 0, label
    assert (np.diff(off[1:m + 1]) >= 0).all(), label
    assert (off[m:] == n_tok).all(), label
    mem = mem[:n_tok]
    assert np.array_equal(np.sort(mem), np.arange(64, 64 * m)), label
    assign = np.empty(n_tok, dtype=np.int64)
    for c in range(1, m):
        seg = mem[off[c]:off[c + 1]]
        assert (np.diff(seg) > 0).all(), (label, c)
        assign[seg - 64] = c
    return assign


def check_step(x, cents_in, cents_out, assign, label, tokens=None):
    """One Lloyd step of the GPU (cents_in -> assign, cents_out) against the
    oracle step from the same centroids. tokens: optional sample of token
    indices whose nearest centroid is recomputed (all when None).
    Returns the number of near-tie tokens."""
    m = cents_in.shape[0]
    ci = cents_in.astype(F64)
    idx = np.arange(len(x)) if tokens is None else np.asarray(tokens)
    o_assign = oc.nearest_centroid(x[idx], ci[1:]) + 1
    g_assign = assign[idx]
    diff = np.nonzero(o_assign != g_assign)[0]
    for i in diff:
        xt = x[idx[i]]
        o, g = o_assign[i], g_assign[i]
        s = lambda c: xt @ ci[c] - 0.5 * ci[c] @ ci[c]
        mag = np.linalg.norm(xt) * (np.linalg.norm(ci[o]) + np.linalg.norm(
            ci[g])) + 0.5 * (ci[o] @ ci[o] + ci[g] @ ci[g])
        assert s(o) - s(g) <= ASSIGN_BAND * mag, (label, idx[i], o, g)
    assert len(diff) <= max(2, 0.01 * len(idx)), (label, len(diff), len(idx))
    # each centroid is the mean of its members (empty: unchanged)
    counts = np.bincount(assign, minlength=m)
    for c in range(1, m):
        if counts[c] == 0:
            assert np.array_equal(cents_out[c], cents_in[c]), (label, c)
            continue
        want = x[assign == c].mean(axis=0)
        tol = CENT_TOL * max(1.0, np.abs(want).max())
        assert np.abs(cents_out[c] - want).max() <= tol, (label, c)
    return len(diff)


def _gpu_and_oracle_step(g, y, iters_done, label):
    """Runs one more GPU step and checks it against the oracle step from the
    GPU's previous centroids."""
    prev = g.cent.cpu().numpy()
    m_arr, off, mem, cents = g.cluster(1)
    ties = 0
    for b, L in enumerate(y["cache_len"]):
        m = int(m_arr[b])
        assert m == oc.cluster_count(int(L), 64, y["n_recent"]), (label, b)
        for rho in range(len(y["retrieval_heads"])):
            if m < 2:
                continue
            lab = f"{label} step {iters_done + 1} b={b} rho={rho}"
            assign = check_tables(m, off[b, rho], mem[b, rho], lab)
            x = _x(y, b, rho, m)
            ties += check_step(x, prev[b, rho, :m], cents[b, rho, :m],
                               assign, lab)
    return ties


@pytest.mark.parametrize("r", [16, 32])
def test_cluster_steps_match_the_oracle(gpu_lib, r):
    lens = [64 * 120 + 17, 64 * 40, 64 * 3 + 5, 100, 64 * 9]
    y = make_decode(_wl(5, max(lens), Hq=4, Hkv=2, ret=(1, 2), window=64,
                        top_k=8, r=r, seed=r), cache_len=lens)
    g = Gpu(gpu_lib, y, r=r)
    print(f"[cluster] r={r} lens={lens}", flush=True)
    ties = 0
    for it in range(3):
        ties += _gpu_and_oracle_step(g, y, it, f"r{r}")
    print(f"[cluster] r={r}: 3 steps, {ties} near-tie tokens", flush=True)


def test_cluster_many_stages_and_chunks(gpu_lib):
    # about 1000 clusters: four LDS stages of centroids in the assignment,
    # 63 chunks in the stable grouping, and a ragged last stage
    L = 64 * 1003 + 9
    y = make_decode(_wl(1, L, Hq=2, Hkv=1, ret=(0,), window=64, top_k=16,
                        seed=3))
    g = Gpu(gpu_lib, y)
    print(f"[cluster] L={L}", flush=True)
    ties = 0
    for it in range(2):
        ties += _gpu_and_oracle_step(g, y, it, "1k")
    print(f"[cluster] 1k clusters: {ties} near-tie tokens", flush=True)


def test_iterations_in_one_call_equal_chained_calls(gpu_lib):
    lens = [64 * 70 + 3, 64 * 33]
    y = make_decode(_wl(2, max(lens), Hq=4, Hkv=1, ret=(0, 3), window=64,
                        top_k=8, seed=5), cache_len=lens)
    a, b = Gpu(gpu_lib, y), Gpu(gpu_lib, y)
    ra = a.cluster(3)
    for _ in range(3):
        rb = b.cluster(1)
    for u, v in zip(ra, rb):
        assert np.array_equal(u, v)


def test_no_step_gives_the_blocks_and_the_block_decode(gpu_lib):
    # iters = 0: the clusters are the blocks, and the clustered decode is
    # the block decode bit for bit (same tokens, tiles, splits and order)
    lens = [64 * 300 + 17, 64 * 71, 777, 65, 1, 64 * 67 + 1]
    y = make_decode(_wl(6, max(lens), Hq=8, Hkv=2, ret=(1, 6), window=300,
                        top_k=12, seed=7), cache_len=lens)
    g = Gpu(gpu_lib, y)
    cent0 = g.cent.clone()
    m, off, mem, cents = g.cluster(0)
    assert torch.equal(g.cent, cent0)
    for b, L in enumerate(lens):
        mm = oc.cluster_count(L, 64, 2)
        assert m[b] == mm
        for rho in range(2):
            assert off[b, rho, :mm + 1].tolist() == [0] + [
                64 * (c - 1) for c in range(1, mm + 1)]
            assert mem[b, rho, :64 * (mm - 1)].tolist() == list(
                range(64, 64 * mm))
    out_c, lse_c, sel_c = g.decode()
    out_b, lse_b, sel_b = gpu_lib.hybrid_attn_decode(
        g.q, g.kc, g.vc, g.cl, y["is_retrieval"], y["window"], g.pq, g.cent,
        y["top_k"], n_recent=2, want_lse=True, want_sel=True)
    torch.cuda.synchronize()
    assert torch.equal(sel_c, sel_b)
    assert torch.equal(out_c.view(torch.int16), out_b.view(torch.int16))
    assert torch.equal(lse_c, lse_b)


def check_clustered_decode(g, y, label):
    """Decode parity given the GPU's clusters."""
    out, lse, sel = g.decode()
    m_arr, off, mem, cents = g.read()
    gsel = sel.cpu().numpy()
    n_ret = len(y["retrieval_heads"])
    clusters = dict(m=m_arr, cents={}, offsets={}, members={})
    for b in range(len(y["cache_len"])):
        for rho in range(n_ret):
            clusters["cents"][(b, rho)] = cents[b, rho].astype(F64)
            clusters["offsets"][(b, rho)] = off[b, rho]
            clusters["members"][(b, rho)] = mem[b, rho]
    args = (bf16_bits(y["q"]), bf16_bits(y["k_cache"]),
            bf16_bits(y["v_cache"]), y["cache_len"], y["is_retrieval"],
            y["window"], y["p_q"], y["p_k"], 64, y["top_k"], clusters)
    ora = oc.clustered_decode(*args, n_recent=y["n_recent"])
    ties, override = [], {}
    G = y["q"].shape[1] // y["k_cache"].shape[1]
    for b, L in enumerate(y["cache_len"]):
        L = int(L)
        n_b, m = -(-L // 64), int(m_arr[b])
        for rho in range(n_ret):
            h = y["retrieval_heads"][rho]
            o_ = off[b, rho]
            empty = lambda c: 1 <= c < m and o_[c + 1] == o_[c]
            row = [int(v) for v in gsel[b, rho] if v >= 0]
            assert row == sorted(set(row)), (label, b, rho)
            req = {0} | set(range(max(0, n_b - 2), n_b))
            assert req <= set(row), (label, b, rho)
            got = [c for c in row if not empty(c)]
            want = ora["sel"][(b, rho)].tolist()
            if got != want:
                # a near-tie at the cut: recompute the candidate scores as
                # the oracle does and check the differing ids
                qt = (y["p_q"][rho].astype(np.float32) @ oracle.bf16_to_f32(
                    bf16_bits(y["q"][b, h]))).astype(np.float32)
                kf = oracle.bf16_to_f32(bf16_bits(y["k_cache"][b, h // G, :L]))
                later = oracle.decode_centroids(kf, y["p_k"][rho], 64, L // 64)
                n_c = max(n_b - 3, 0)
                sc = {}
                for c in range(1, n_c + 1):
                    if empty(c):
                        continue
                    cv = cents[b, rho, c] if c < m else later[c]
                    sc[c] = float(np.float32(cv.astype(np.float32) @ qt))
                srt = sorted(sc.values(), reverse=True)
                k = y["top_k"]
                s_k, s_k1 = srt[k - 1], srt[k]
                assert abs(s_k - s_k1) <= parity.TIE_BAND * abs(s_k), \
                    (label, b, rho, s_k, s_k1)
                for c in set(got) ^ set(want):
                    assert c in sc and abs(sc[c] - s_k) <= \
                        parity.TIE_BAND * abs(s_k), (label, b, rho, c)
                ties.append((b, rho))
                override[(b, rho)] = got
    parity.assert_tie_rate(ties, len(y["cache_len"]) * n_ret, label)
    if override:
        ora = oc.clustered_decode(*args, n_recent=y["n_recent"],
                                  sel_override=override)
    o_g = parity.bf16_to_f32(out)
    l_g = lse.cpu().numpy()
    worst = 0.0
    for b in range(len(y["cache_len"])):
        for h in range(o_g.shape[1]):
            err = parity.max_abs(o_g[b, h], ora["out"][b, h])
            assert err <= parity.OUT_TOL, (label, b, h, err)
            lerr = abs(l_g[b, h] - ora["lse"][b, h])
            assert lerr <= parity.LSE_TOL_BF16_SUM, (label, b, h, lerr)
            worst = max(worst, lerr)
    print(f"[cluster] decode {label}: lse {worst:.2e}, ties {len(ties)}",
          flush=True)


@pytest.mark.parametrize("top_k", [1, 12, 65])
def test_clustered_decode_matches_the_oracle(gpu_lib, top_k):
    lens = [64 * 200 + 17, 64 * 71, 777, 65, 64 * 67 + 1]
    y = make_decode(_wl(5, max(lens), Hq=8, Hkv=2, ret=(1, 6), window=300,
                        top_k=top_k, seed=11), cache_len=lens)
    g = Gpu(gpu_lib, y)
    g.cluster(2)
    check_clustered_decode(g, y, f"k={top_k}")


def test_clustered_decode_after_appends(gpu_lib):
    # The caches grow by 150 tokens after the clustering: two and three
    # blocks leave the recent window and become ordinary candidates, with the
    # block centroids the appends keep.
    lens = [64 * 90 + 30, 64 * 40 + 63]
    y = make_decode(_wl(2, max(lens) + 200, Hq=4, Hkv=1, ret=(0, 2),
                        window=128, top_k=6, seed=13), cache_len=lens,
                    Lmax=max(lens) + 200)
    g = Gpu(gpu_lib, y)
    g.cluster(2)
    gen = torch.Generator().manual_seed(5)
    for _ in range(150):
        kn = torch.randn((2, 1, 128), generator=gen).to(torch.bfloat16)
        vn = torch.randn((2, 1, 128), generator=gen).to(torch.bfloat16)
        gpu_lib.decode_append(g.kc, g.vc, g.cl, kn.cuda(), vn.cuda(),
                              y["is_retrieval"], g.pk, g.cent)
    torch.cuda.synchronize()
    y = dict(y)
    y["k_cache"], y["v_cache"] = g.kc.cpu(), g.vc.cpu()
    y["cache_len"] = g.cl.cpu().numpy()
    assert y["cache_len"].tolist() == [L + 150 for L in lens]
    check_clustered_decode(g, y, "appended")


def test_clustered_decode_full_size_sampled(gpu_lib):
    # 32 sequences x 256K cached tokens, 5 retrieval heads, top-64 clusters,
    # two Lloyd steps. Checked: every (sequence, head)'s tables; for two
    # (sequence, head) pairs, the nearest centroid of 4096 sampled tokens at
    # the second step and every centroid as the mean of its members; the
    # decode choice and outputs of four sequences (run alone, and equal to
    # the same sequences of the whole batch).
    from workloads import DECODE_32x256K as w
    y = make_decode(w, device="cuda")
    print("[cluster] full size: clustering", flush=True)
    g = Gpu(gpu_lib, y)
    g.cluster(1)
    prev = g.cent.cpu().numpy()
    m_arr, off, mem, cents = g.cluster(1)
    for b in range(w.batch):
        m = int(m_arr[b])
        for rho in range(w.n_ret):
            check_tables(m, off[b, rho], mem[b, rho], f"full b={b} rho={rho}")
    out_all = g.decode()[0]
    seqs = [0, 7, 19, 31]
    sub = dict(y)
    for key in ("q", "k_cache", "v_cache"):
        sub[key] = y[key][seqs].cpu()
    sub["cache_len"] = y["cache_len"][seqs]
    rng = np.random.default_rng(0)
    for b, rho in ((0, 0), (3, w.n_ret - 1)):
        m = int(m_arr[seqs[b]])
        assign = check_tables(m, off[seqs[b], rho], mem[seqs[b], rho], "full")
        x = _x(sub, b, rho, m)
        toks = rng.choice(len(x), 4096, replace=False)
        check_step(x, prev[seqs[b], rho, :m], cents[seqs[b], rho, :m], assign,
                   f"full b={seqs[b]} rho={rho}", tokens=toks)
    print("[cluster] full size: decode", flush=True)
    gs = Gpu.__new__(Gpu)
    gs.rtp, gs.y, gs.r = gpu_lib, sub, 16
    gs.q, gs.kc, gs.vc = g.q[seqs], g.kc[seqs], g.vc[seqs]
    gs.cl, gs.pk, gs.pq = g.cl[seqs], g.pk, g.pq
    gs.cent = g.cent[seqs].contiguous()
    gs.tables = tuple(t[seqs].contiguous() for t in g.tables)
    check_clustered_decode(gs, sub, "full")
    out_sub = gs.decode()[0]
    assert torch.equal(out_sub.view(torch.int16), out_all[seqs].view(torch.int16))


def test_clustered_decode_rank_32(gpu_lib):
    # r = 32: the selection's general scoring loop (with the empty-cluster
    # check) and two 16-row halves per projection tile
    lens = [64 * 150 + 40, 64 * 33 + 1]
    y = make_decode(_wl(2, max(lens), Hq=4, Hkv=1, ret=(0, 2), window=128,
                        top_k=9, r=32, seed=17), cache_len=lens)
    g = Gpu(gpu_lib, y, r=32)
    for it in range(2):
        _gpu_and_oracle_step(g, y, it, "r32 decode")
    check_clustered_decode(g, y, "r32")
