"""GPU parity at the benchmarked sizes, in the benchmarked launch configuration.

The library is called exactly as ``bench.py`` calls it (same entry points, one
workspace sized by the library, inputs drawn on the GPU). The oracle then
checks what it can finish at these sizes:

* 32K layer: every selection row of every retrieval head, and all heads'
  outputs and LSE on sampled query blocks;
* 128K layer with needles: every selection row of all 5 retrieval heads, and
  outputs of sampled query blocks of every head (the first, the last, the
  blocks around the needle boundary S/2 and random ones);
* 1M all-sparse layer: a stratified sample of at least 256 selection rows of
  every one of the 23 retrieval heads (one random row per stratum of 64
  rows, plus the first rows, the rows around S/2 and the last), and outputs
  of sampled (head, query block) pairs;
* decode, 32 sequences of 256K tokens: sampled sequences, every head.

One GPU run of a workload serves all the tests of that workload (the
results are kept until the next workload runs).
"""
import numpy as np
import pytest
import torch

import oracle
from tests import parity
from workloads import (PREFILL_32K, PREFILL_128K, PREFILL_1M, DECODE_32x256K,
                       make_prefill, make_decode, bf16_bits,
                       retrieval_heads_for)

pytestmark = pytest.mark.gpu


def _host_bits(t, index):
    """uint16 copy of t with only t[i], i in index, filled (the rest of the
    buffer is never touched, so it costs no host memory)."""
    arr = np.empty(tuple(t.shape), dtype=np.uint16)
    for i in index:
        arr[i] = bf16_bits(t[i])
    return arr


def _run_prefill(rtp, x, w):
    dev = "cuda"
    pq = torch.from_numpy(x["p_q"]).to(dev)
    pk = torch.from_numpy(x["p_k"]).to(dev)
    ws = torch.empty(rtp.prefill_workspace_bytes(w.S, w.Hq, w.Hkv,
                                                 x["is_retrieval"], w.r,
                                                 w.top_k),
                     dtype=torch.uint8, device=dev)
    out = torch.empty_like(x["q"])
    res = rtp.hybrid_attn_prefill(x["q"], x["k"], x["v"], x["is_retrieval"],
                                  w.window, pq, pk, w.top_k, r=w.r, ws=ws,
                                  out=out, want_lse=True, want_sel=True)
    torch.cuda.synchronize()
    del ws
    return res


_RUN = {}


def gpu_run(rtp, w):
    """Inputs and GPU results of workload w (one run, kept for its tests)."""
    if _RUN.get("name") != w.name:
        _RUN.clear()
        torch.cuda.empty_cache()
        print(f"[full-size] {w.name}: GPU run", flush=True)
        x = make_prefill(w, device="cuda")
        out, lse, sel, cnt = _run_prefill(rtp, x, w)
        _RUN.update(name=w.name, x=x, out=out, lse=lse,
                    sel=sel.cpu().numpy(), cnt=cnt.cpu().numpy(), bits={})
    return _RUN


def _bits(run, key, idx):
    """Host bf16 bits of run["x"][key][i] for i in idx (cached per index)."""
    t = run["x"][key]
    cache = run["bits"].setdefault(key, np.empty(tuple(t.shape), np.uint16))
    have = run["bits"].setdefault(key + "_have", set())
    for i in idx:
        if i not in have:
            cache[i] = bf16_bits(t[i])
            have.add(i)
    return cache


def check_selection(rtp, w, rows_of_rho):
    """Selection rows of the given retrieval heads against the oracle.

    rows_of_rho: dict rho -> query blocks. Returns the logged ties."""
    run = gpu_run(rtp, w)
    x = run["x"]
    ret = list(x["retrieval_heads"])
    G = w.Hq // w.Hkv
    ties = []
    for rho, rows in sorted(rows_of_rho.items()):
        h = ret[rho]
        rows = sorted(set(rows))
        qb_bits = _bits(run, "q", [h])
        kb_bits = _bits(run, "k", [h // G])
        ora = oracle.hybrid_prefill(qb_bits, kb_bits, kb_bits,
                                    x["is_retrieval"], w.window, x["p_q"],
                                    x["p_k"], 64, w.top_k, heads=[h],
                                    query_blocks=[], sel_rows=rows)
        fn = parity.prefill_rows_fn(x, qb_bits, kb_bits, rho, h)
        t = parity.compare_selection(
            run["sel"][rho][rows], run["cnt"][rho][rows], ora["sel"][rho][rows],
            ora["sel_count"][rho][rows], ora["kth"][rho][rows],
            lambda i, fn=fn, rows=rows: fn(rows[i]),
            parity.prefill_required(lambda i, rows=rows: rows[i]),
            f"{w.name} rho={rho}")
        ties += t
        print(f"[full-size] {w.name} rho={rho} (head {h}): {len(rows)} rows "
              f"identical except {len(t)} logged ties", flush=True)
    return ties


def check_outputs(rtp, w, qbs, heads=None):
    """Outputs and LSE of sampled query blocks, under the GPU's selection
    (identical to the oracle's except at logged ties, checked separately)."""
    run = gpu_run(rtp, w)
    x = run["x"]
    heads = list(range(w.Hq)) if heads is None else list(heads)
    G = w.Hq // w.Hkv
    groups = sorted({h // G for h in heads})
    print(f"[full-size] {w.name}: outputs qbs={sorted(qbs)} heads={heads}",
          flush=True)
    qb_bits = _bits(run, "q", heads)
    kb_bits = _bits(run, "k", groups)
    vb_bits = _bits(run, "v", groups)
    sel, cnt = run["sel"], run["cnt"]
    override = {rho: {qb: sel[rho, qb, :cnt[rho, qb]] for qb in qbs}
                for rho in range(len(x["retrieval_heads"]))}
    ora = oracle.hybrid_prefill(qb_bits, kb_bits, vb_bits, x["is_retrieval"],
                                w.window, x["p_q"], x["p_k"], 64, w.top_k,
                                sel_override=override, heads=heads,
                                query_blocks=sorted(qbs))
    out, lse = run["out"], run["lse"]
    worst = 0.0
    lworst = {"window": 0.0, "sparse": 0.0}
    for h in heads:
        for qb in qbs:
            s = slice(qb * 64, min(w.S, qb * 64 + 64))
            o_g = out[h, s].float().cpu().numpy()
            err = parity.max_abs(o_g, ora["out"][h, s])
            assert err <= parity.OUT_TOL, (w.name, h, qb, err)
            worst = max(worst, err)
            lw = parity.check_prefill_lse(
                lse[h:h + 1, s].cpu().numpy(), ora["lse"][h:h + 1, s],
                x["is_retrieval"][h:h + 1], f"{w.name} h={h} qb={qb}")
            for key in lworst:
                lworst[key] = max(lworst[key], lw[key])
    print(f"[full-size] {w.name}: max |dO| {worst:.2e}, max |dLSE| window "
          f"{lworst['window']:.2e} sparse {lworst['sparse']:.2e}", flush=True)


def _qbs(n_b, extra, seed):
    rng = np.random.default_rng(seed)
    fixed = {0, 1, n_b // 2 - 1, n_b // 2, n_b - 1}
    return sorted(fixed | set(int(i) for i in rng.choice(n_b, extra,
                                                         replace=False)))


def _stratified_rows(n_b, seed, stride=64):
    """One random row per stratum of `stride` rows, plus the first rows, the
    rows around the needle boundary n_b/2 and the last row."""
    rng = np.random.default_rng(seed)
    rows = {0, 1, 2, n_b // 2 - 1, n_b // 2, n_b // 2 + 1, n_b - 2, n_b - 1}
    for lo in range(0, n_b, stride):
        rows.add(int(rng.integers(lo, min(n_b, lo + stride))))
    return sorted(rows)


def test_prefill_32k_every_selection_row_and_sampled_outputs(gpu_lib):
    w = PREFILL_32K
    n_b = w.S // 64
    ties = check_selection(gpu_lib, w, {rho: range(n_b)
                                        for rho in range(w.n_ret)})
    parity.assert_tie_rate(ties, w.n_ret * n_b, w.name)
    check_outputs(gpu_lib, w, _qbs(n_b, 3, 1))


def test_prefill_128k_needles_every_selection_row(gpu_lib):
    w = PREFILL_128K
    n_b = w.S // 64
    ties = check_selection(gpu_lib, w, {rho: range(n_b)
                                        for rho in range(w.n_ret)})
    parity.assert_tie_rate(ties, w.n_ret * n_b, w.name)


def test_prefill_128k_needles_sampled_outputs(gpu_lib):
    w = PREFILL_128K
    check_outputs(gpu_lib, w, _qbs(w.S // 64, 3, 2))


@pytest.mark.parametrize("part", range(4))
def test_prefill_1m_all_sparse_selection_rows(gpu_lib, part):
    # 23 retrieval heads in four parts; each head gets its own stratified
    # sample of at least 256 rows
    w = PREFILL_1M
    n_b = w.S // 64
    rhos = [rho for rho in range(w.n_ret) if rho % 4 == part]
    rows = {rho: _stratified_rows(n_b, 100 + rho) for rho in rhos}
    ties = check_selection(gpu_lib, w, rows)
    parity.assert_tie_rate(ties, sum(len(r) for r in rows.values()), w.name)


def test_prefill_1m_all_sparse_sampled_outputs(gpu_lib):
    w = PREFILL_1M
    n_b = w.S // 64
    ret = list(retrieval_heads_for(w.Hq, w.n_ret, w.seed, w.retrieval_heads))
    swa = [h for h in range(w.Hq) if h not in ret]
    heads = sorted({ret[0], ret[-1], swa[0], swa[-1]})
    check_outputs(gpu_lib, w, _qbs(n_b, 2, 3), heads=heads)


def _fresh_check(rtp, w, qbs):
    """Whole selection and sampled outputs of a small irregular workload."""
    _RUN.clear()
    n_b = w.n_blocks
    ties = check_selection(rtp, w, {rho: range(n_b)
                                    for rho in range(w.n_ret)})
    parity.assert_tie_rate(ties, w.n_ret * n_b, w.name)
    check_outputs(rtp, w, qbs)
    _RUN.clear()


def test_prefill_past_the_stream_fork_threshold(gpu_lib):
    # beyond 4096 blocks the window heads run on the auxiliary stream while
    # the indexer runs; ragged, two KV groups, one retrieval head
    from workloads import PrefillWorkload
    w = PrefillWorkload("fork_threshold", S=64 * 4100 + 7, Hq=4, Hkv=2, d=128,
                        n_ret=1, window=300, r=16, block=64, top_k=8,
                        retrieval_heads=(1,))
    n_b = w.n_blocks
    _fresh_check(gpu_lib, w, [0, 1, 2047, 4095, 4096, n_b - 2, n_b - 1])


def test_forked_prefill_runs_after_earlier_work_on_the_callers_stream(gpu_lib):
    # Past 4096 blocks the window heads run on the library's auxiliary
    # stream. V = 1 is produced by a kernel on a side stream right before
    # the call on that stream: every output is exactly 1 only if all heads
    # waited for it, and the next kernel on the stream sees the outputs.
    from workloads import PrefillWorkload
    _RUN.clear()
    w = PrefillWorkload("fork_order", S=64 * 4097 + 3, Hq=4, Hkv=2, d=128,
                        n_ret=1, window=256, r=16, block=64, top_k=4,
                        retrieval_heads=(2,))
    x = make_prefill(w, device="cuda")
    pq = torch.from_numpy(x["p_q"]).cuda()
    pk = torch.from_numpy(x["p_k"]).cuda()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        for _ in range(2):
            v1 = torch.empty_like(x["k"])
            v1.copy_(x["k"]).mul_(0).add_(1)
            out = gpu_lib.hybrid_attn_prefill(x["q"], x["k"], v1,
                                              x["is_retrieval"], w.window, pq,
                                              pk, w.top_k)
            bad = (out != 1).sum()
            assert int(bad.item()) == 0


def test_decode_32x256k_sampled_sequences(gpu_lib):
    _RUN.clear()
    torch.cuda.empty_cache()
    w = DECODE_32x256K
    print(f"[full-size] {w.name}", flush=True)
    y = make_decode(w, device="cuda")
    dev = "cuda"
    cl = torch.from_numpy(y["cache_len"]).to(dev)
    pq = torch.from_numpy(y["p_q"]).to(dev)
    pk = torch.from_numpy(y["p_k"]).to(dev)
    cent = gpu_lib.build_centroids(y["k_cache"], cl, y["is_retrieval"], pk)
    ws = torch.empty(gpu_lib.decode_workspace_bytes(w.batch, w.L, w.Hq, w.Hkv,
                                                    y["is_retrieval"], w.r,
                                                    w.top_k, w.n_recent),
                     dtype=torch.uint8, device=dev)
    out = torch.empty_like(y["q"])
    out, lse, sel = gpu_lib.hybrid_attn_decode(
        y["q"], y["k_cache"], y["v_cache"], cl, y["is_retrieval"], w.window,
        pq, cent, w.top_k, n_recent=w.n_recent, ws=ws, out=out, want_lse=True,
        want_sel=True)
    torch.cuda.synchronize()
    seqs = [0, 13, w.batch - 1]
    args = (bf16_bits(y["q"]), _host_bits(y["k_cache"], seqs),
            _host_bits(y["v_cache"], seqs), y["cache_len"], y["is_retrieval"],
            w.window, y["p_q"], y["p_k"], 64, w.top_k, w.n_recent)
    ora = oracle.hybrid_decode(*args, seqs=seqs)
    gsel = sel.cpu().numpy()
    gcent = cent.cpu().numpy()
    ret = list(y["retrieval_heads"])
    override, n_ties = {}, 0
    for b in seqs:
        L = int(y["cache_len"][b])
        n_full, n_b = L // 64, -(-L // 64)
        for rho, h in enumerate(ret):
            c_o = ora["centroids"][(b, rho)]
            assert np.abs(gcent[b, rho, :n_full] - c_o).max() <= \
                1e-5 * max(np.abs(c_o).max(), 1.0), (b, rho)
            qt = y["p_q"][rho] @ oracle.bf16_to_f32(bf16_bits(y["q"][b, h]))
            g = gsel[b, rho]
            gcnt = int((g >= 0).sum())
            ties = parity.compare_selection(
                g[None], np.array([gcnt]), ora["sel"][b, rho][None],
                ora["sel_count"][b, rho][None], ora["kth"][b, rho][None],
                parity.decode_scores_fn(c_o, qt, n_b, w.n_recent),
                parity.decode_required(n_b, w.n_recent), f"b={b} rho={rho}")
            if ties:
                override[(b, rho)] = g[:gcnt]
                n_ties += len(ties)
    parity.assert_tie_rate(list(override), len(seqs) * len(ret), w.name)
    if override:  # tie rows: attend under the GPU's own (valid) choice
        ora = oracle.hybrid_decode(*args, seqs=seqs, sel_override=override)
    o_g = out.float().cpu().numpy()
    l_g = lse.cpu().numpy()
    worst = lworst = 0.0
    for b in seqs:
        for h in range(w.Hq):
            err = parity.max_abs(o_g[b, h], ora["out"][b, h])
            assert err <= parity.OUT_TOL, (b, h, err)
            lerr = abs(l_g[b, h] - ora["lse"][b, h])
            assert lerr <= parity.LSE_TOL_BF16_SUM, (b, h, lerr)
            worst, lworst = max(worst, err), max(lworst, lerr)
    print(f"[full-size] {w.name}: max |dO| {worst:.2e}, max |dLSE| "
          f"{lworst:.2e}, ties {n_ties}", flush=True)
