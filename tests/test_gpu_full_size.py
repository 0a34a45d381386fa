"""GPU parity at the benchmarked sizes, in the benchmarked launch configuration.

The library is called exactly as ``bench.py`` calls it (same entry points, one
workspace sized by the library, inputs drawn on the GPU). The oracle then
checks what it can finish in seconds at these sizes:

* 32K layer: every selection row of every retrieval head, and all heads'
  outputs and LSE on sampled query blocks;
* 128K layer with needles and the 1M all-sparse layer: selection rows and
  outputs of sampled (head, query block) pairs, including the first, the
  last and the blocks around the needle boundary S/2;
* decode, 32 sequences of 256K tokens: sampled sequences, every head.
"""
import numpy as np
import pytest
import torch

import oracle
from tests import parity
from workloads import (PREFILL_32K, PREFILL_128K, PREFILL_1M, DECODE_32x256K,
                       make_prefill, make_decode, bf16_bits)

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
    return res


def sampled_check(rtp, w, qbs, heads=None, all_sel_rows=False):
    print(f"[full-size] {w.name}: qbs={sorted(qbs)} heads={heads}", flush=True)
    x = make_prefill(w, device="cuda")
    out, lse, sel, cnt = _run_prefill(rtp, x, w)
    ret = list(x["retrieval_heads"])
    heads = list(range(w.Hq)) if heads is None else list(heads)
    groups = sorted({h // (w.Hq // w.Hkv) for h in heads})
    qb_bits = _host_bits(x["q"], heads)
    kb_bits = _host_bits(x["k"], groups)
    vb_bits = _host_bits(x["v"], groups)
    n_b = -(-w.S // 64)
    rows = range(n_b) if all_sel_rows else sorted(qbs)
    ora = oracle.hybrid_prefill(qb_bits, kb_bits, vb_bits, x["is_retrieval"],
                                w.window, x["p_q"], x["p_k"], 64, w.top_k,
                                heads=heads, query_blocks=sorted(qbs),
                                sel_rows=rows)
    gsel, gcnt = sel.cpu().numpy(), cnt.cpu().numpy()
    ties = []
    for rho, h in enumerate(ret):
        if h not in heads:
            continue
        fn = parity.prefill_rows_fn(x, qb_bits, kb_bits, rho, h)
        r = list(rows)
        ties += parity.compare_selection(
            gsel[rho][r], gcnt[rho][r], ora["sel"][rho][r],
            ora["sel_count"][rho][r], ora["kth"][rho][r],
            lambda i, fn=fn, r=r: fn(r[i]), f"{w.name} rho={rho}")
    if ties:  # attend under the GPU's own (equally valid) selection
        override = {rho: {qb: gsel[rho, qb, :gcnt[rho, qb]] for qb in qbs}
                    for rho in range(len(ret))}
        ora = oracle.hybrid_prefill(qb_bits, kb_bits, vb_bits,
                                    x["is_retrieval"], w.window, x["p_q"],
                                    x["p_k"], 64, w.top_k,
                                    sel_override=override, heads=heads,
                                    query_blocks=sorted(qbs))
    worst = 0.0
    for h in heads:
        for qb in qbs:
            s = slice(qb * 64, min(w.S, qb * 64 + 64))
            o_g = out[h, s].float().cpu().numpy()
            err = parity.max_abs(o_g, ora["out"][h, s])
            lerr = parity.max_abs(lse[h, s].cpu().numpy(), ora["lse"][h, s])
            assert err <= parity.OUT_TOL, (w.name, h, qb, err)
            assert lerr <= parity.LSE_TOL, (w.name, h, qb, lerr)
            worst = max(worst, err)
    print(f"[full-size] {w.name}: max |dO| {worst:.2e}, ties {len(ties)}",
          flush=True)
    return ties


def _qbs(n_b, extra, seed):
    rng = np.random.default_rng(seed)
    fixed = {0, 1, n_b // 2 - 1, n_b // 2, n_b - 1}
    return sorted(fixed | set(int(i) for i in rng.choice(n_b, extra,
                                                         replace=False)))


def test_prefill_32k_every_selection_row_and_sampled_outputs(gpu_lib):
    n_b = PREFILL_32K.S // 64
    sampled_check(gpu_lib, PREFILL_32K, _qbs(n_b, 3, 1), all_sel_rows=True)


def test_prefill_128k_needles_sampled(gpu_lib):
    n_b = PREFILL_128K.S // 64
    sampled_check(gpu_lib, PREFILL_128K, _qbs(n_b, 3, 2))


def test_prefill_1m_all_sparse_sampled(gpu_lib):
    w = PREFILL_1M
    n_b = w.S // 64
    from workloads import retrieval_heads_for
    ret = list(retrieval_heads_for(w.Hq, w.n_ret, w.seed, w.retrieval_heads))
    swa = [h for h in range(w.Hq) if h not in ret]
    heads = sorted({ret[0], ret[-1], swa[0], swa[-1]})
    sampled_check(gpu_lib, w, _qbs(n_b, 2, 3), heads=heads)


def test_prefill_past_the_stream_fork_threshold(gpu_lib):
    # beyond 4096 blocks the window heads run on the auxiliary stream while
    # the indexer runs; ragged, two KV groups, one retrieval head
    from workloads import PrefillWorkload
    w = PrefillWorkload("fork_threshold", S=64 * 4100 + 7, Hq=4, Hkv=2, d=128,
                        n_ret=1, window=300, r=16, block=64, top_k=8,
                        retrieval_heads=(1,))
    n_b = w.n_blocks
    sampled_check(gpu_lib, w, [0, 1, 2047, 4095, 4096, n_b - 2, n_b - 1])


def test_forked_prefill_runs_after_earlier_work_on_the_callers_stream(gpu_lib):
    # Past 4096 blocks the window heads run on the library's auxiliary
    # stream. V = 1 is produced by a kernel on a side stream right before
    # the call on that stream: every output is exactly 1 only if all heads
    # waited for it, and the next kernel on the stream sees the outputs.
    from workloads import PrefillWorkload
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
    ora = oracle.hybrid_decode(bf16_bits(y["q"]), _host_bits(y["k_cache"], seqs),
                               _host_bits(y["v_cache"], seqs), y["cache_len"],
                               y["is_retrieval"], w.window, y["p_q"], y["p_k"],
                               64, w.top_k, w.n_recent, seqs=seqs)
    gsel = sel.cpu().numpy()
    gcent = cent.cpu().numpy()
    ret = list(y["retrieval_heads"])
    skip = set()
    for b in seqs:
        n_full = int(y["cache_len"][b]) // 64
        for rho, h in enumerate(ret):
            c_o = ora["centroids"][(b, rho)]
            assert np.abs(gcent[b, rho, :n_full] - c_o).max() <= \
                1e-5 * max(np.abs(c_o).max(), 1.0), (b, rho)
            qt = y["p_q"][rho] @ oracle.bf16_to_f32(bf16_bits(y["q"][b, h]))
            g = gsel[b, rho]
            ties = parity.compare_selection(
                g[None], np.array([int((g >= 0).sum())]),
                ora["sel"][b, rho][None], ora["sel_count"][b, rho][None],
                ora["kth"][b, rho][None],
                lambda _, c_o=c_o, qt=qt: c_o[1:] @ qt.astype(np.float32),
                f"b={b} rho={rho}")
            if ties:
                skip.add((b, h))
    assert len(skip) <= 1, skip
    o_g = out.float().cpu().numpy()
    l_g = lse.cpu().numpy()
    worst = 0.0
    for b in seqs:
        for h in range(w.Hq):
            if (b, h) in skip:
                continue
            err = parity.max_abs(o_g[b, h], ora["out"][b, h])
            assert err <= parity.OUT_TOL, (b, h, err)
            assert abs(l_g[b, h] - ora["lse"][b, h]) <= parity.LSE_TOL, (b, h)
            worst = max(worst, err)
    print(f"[full-size] {w.name}: max |dO| {worst:.2e}", flush=True)
