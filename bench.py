#!/usr/bin/env python3
"""Benchmark of headwise hybrid attention on one MI355X.

One step = one call of rtp_hybrid_attn_prefill on the 128K-token workload
(one attention layer at Qwen3-30B-A3B shape: 32 query / 4 KV heads, d = 128,
5 retrieval heads with the r = 16 indexer, 27 window heads with w = 8192,
block 64, top-128 blocks, planted needle blocks): the indexer (projection,
block scores, top-k), the V transpose and the attention kernel. Inputs are
synthetic and resident in HBM before timing starts.

The same run also measures, as secondary figures: the 1M-token all-sparse
prefill, the 32K prefill, a decode step of 32 sequences x 256K cached tokens,
and the dense causal kernel of the same library on the 128K inputs. The CPU
oracle is timed on a bounded sample of the 128K workload.

Prints ONE JSON line. Usage: python bench.py [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "hybrid-attn prefill tokens/s at 128K & 1M; decode tok/s; % bf16 MFMA peak"

# HBM bytes per launch, from two rocprofv3 --pmc runs (FETCH_SIZE, then
# WRITE_SIZE) of the leg named, with --copy-probe-gib 1: each counter is
# divided by what it reads per byte of that run's 1 GiB plain device copy
# (0.5 for FETCH_SIZE, 1.0 for WRITE_SIZE on MI355X). A figure is valid only
# for the kernel source it was measured on: sha256 over the listed sources
# and the hipcc flags the build gives the kernel's file. After any change it
# is reported as null.
_K = "long_context_sparse_head_amd/csrc/"
COUNTERS = {
    # bench.py --only-main --no-cpu-baseline --steps 3 --warmup 1
    "attn_window@128k": {
        "kernel": "attn_window", "unit": "attn_window.hip",
        "sources": [_K + "attn_window.hip", _K + "attn_core.h"],
        "sha256": "e988f16308a9848a871682a27ea745cd9d6d1a288e861fe66a4fd55897294521",
        "fetch_bytes": 2935521280, "write_bytes": 906108211},
    "attn_sparse@128k": {
        "kernel": "attn_sparse", "unit": "attn.hip",
        "sources": [_K + "attn.hip", _K + "attn_core.h"],
        "sha256": "834f4571ea4b656c0830fac12fb27fe7456b9715abdd45b7b2f643ce33e3f866",
        "fetch_bytes": 16634910925,
        "write_bytes": 167957811},
    # bench.py --leg 1m --steps 2 --warmup 1
    "attn_sparse@1m": {
        "kernel": "attn_sparse", "unit": "attn.hip",
        "sources": [_K + "attn.hip", _K + "attn_core.h"],
        "sha256": "834f4571ea4b656c0830fac12fb27fe7456b9715abdd45b7b2f643ce33e3f866",
        "fetch_bytes": 2409851323392,
        "write_bytes": 6185473024},
}
_IDX = {"unit": "indexer.hip",
        "sources": [_K + "indexer.hip", _K + "proj.h", _K + "select.h"],
        "sha256": "a641ea7d7fc242ba52532275e7c229d901a796f838bba88284e9fe2b45e1acdc"}
_CL = {"unit": "cluster.hip", "sources": [_K + "cluster.hip", _K + "proj.h"],
       "sha256": "4909d7ada22d4370f545ea56ee46ba2f0a1e014964cd583820e60cf8a796a1c7"}
_DEC = {"unit": "decode.hip", "sources": [_K + "decode.hip", _K + "select.h"],
        "sha256": "baf70ffab5a270962dfac5930a881915017b3b38de9b3f542797acb1c77b26aa"}
for _base, _key, _kern, _f, _w in (
        # bench.py --only-main --no-cpu-baseline --steps 3 --warmup 1
        (_IDX, "proj_keys@128k", "proj_keys", 68072499, 41943040),
        (_IDX, "proj_qmeans@128k", "proj_qmeans", 168183706, 656608),
        (_IDX, "block_scores@128k", "block_scores", 263814477, 42334682),
        (_IDX, "topk@128k", "topk", 43118182, 5898240),
        # bench.py --leg 1m --steps 2 --warmup 1
        (_IDX, "proj_keys@1m", "proj_keys", 1090001632, 1543503968),
        (_IDX, "proj_qmeans@1m", "proj_qmeans", 6175660384, 24130680),
        (_IDX, "score_select@1m", "score_select", 57249297440, 14480385896),
        # bench.py --leg cluster --steps 4 --warmup 1 (per launch: one
        # projection and one Lloyd step's kernels)
        (_CL, "cl_project@cluster", "cl_project", 10740339507, 2682495181),
        (_CL, "cl_assign@cluster", "cl_assign", 3018200269, 1475449651),
        (_CL, "cl_update@cluster", "cl_update", 5420282880, 31043072),
        (_DEC, "dec_attn_retrieval@cluster", "dec_attn_retrieval", 523299430,
         698573),
        # bench.py --leg decode --steps 4 --warmup 1
        (_DEC, "dec_attn_window@decode", "dec_attn_window", 539505843,
         3761872),
        (_DEC, "dec_attn_retrieval@decode", "dec_attn_retrieval", 340548365,
         697123),
        (_DEC, "dec_select@decode", "dec_select", 42693939, 52480),
        (_DEC, "dec_merge@decode", "dec_merge", 4352205, 262144)):
    COUNTERS[_key] = dict(_base, kernel=_kern, fetch_bytes=_f, write_bytes=_w)
TRAFFIC_KEY = "attn_window@128k"


def kernel_sources_sha256(entry):
    import hashlib
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_rtp_build_flags", os.path.join(ROOT, "long_context_sparse_head_amd",
                                         "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    flags = b.HIPFLAGS + b.EXTRA_FLAGS.get(entry["unit"], [])
    h = hashlib.sha256()
    for src in entry["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    h.update(" ".join(flags).encode())
    return h.hexdigest()


def counter_bytes(key):
    """(fetch, write) bytes per launch, or None once the source changed."""
    e = COUNTERS[key]
    if e["sha256"] is None or kernel_sources_sha256(e) != e["sha256"]:
        return None
    return e["fetch_bytes"], e["write_bytes"]


def measured_traffic():
    fw = counter_bytes(TRAFFIC_KEY)
    return None if fw is None else fw[0] + fw[1]


def hbm_counters(leg, ks):
    """Counter bytes of this leg's kernels and the rate they imply at the
    kernel times measured in this run."""
    out = {}
    for key, e in COUNTERS.items():
        if not key.endswith("@" + leg):
            continue
        fw = counter_bytes(key)
        t = ks.get(e["kernel"])
        if fw is None or not t:
            out[key] = None
            continue
        out[key] = {"fetch_gb": fw[0] / 1e9, "write_gb": fw[1] / 1e9,
                    "gbs": (fw[0] + fw[1]) / (t["ms_per_launch"] / 1e3) / 1e9}
    return out


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------ accounting
def prefill_pairs(S, Hq, is_ret, window, sel_cnt_np):
    """Executed (query, key) pairs: causal-, window- and selection-exact."""
    i = np.arange(S, dtype=np.int64)
    swa_per_head = int(np.minimum(i + 1, window).sum())
    n_swa = int((np.asarray(is_ret) == 0).sum())
    ret = 0
    n_b = -(-S // 64)
    last = S - 64 * (n_b - 1)
    for rho in range(sel_cnt_np.shape[0]):
        cnt = sel_cnt_np[rho].astype(np.int64)
        diag = np.full(n_b, 64 * 65 // 2, dtype=np.int64)
        diag[-1] = last * (last + 1) // 2
        rows = np.full(n_b, 64, dtype=np.int64)
        rows[-1] = last
        ret += int(((cnt - 1) * 64 * rows + diag).sum())
    return n_swa * swa_per_head, ret


def kernel_stats(records, steps):
    out = {}
    for name, ms in records:
        d = out.setdefault(name, {"launches": 0, "ms_total": 0.0})
        d["launches"] += 1
        d["ms_total"] += ms
    for d in out.values():
        d["ms_per_launch"] = d["ms_total"] / d["launches"]
        d["ms_per_step"] = d["ms_total"] / steps
    return out


# ------------------------------------------------------------ GPU legs
def bench_prefill(rtp, torch, w, steps, warmup, dense=False, full=False,
                  leg=None):
    """dense: every head causal-full (rtp_dense_attn_prefill); full:
    retrieval heads causal-full, streaming heads windowed, with the decode
    centroids as an epilogue (rtp_headwise_prefill, RTP_RETRIEVAL_FULL)."""
    from workloads import make_prefill
    dev = "cuda"
    t0 = time.time()
    x = make_prefill(w, device=dev)
    pq = torch.from_numpy(x["p_q"]).to(dev)
    pk = torch.from_numpy(x["p_k"]).to(dev)
    S, Hq, Hkv = w.S, w.Hq, w.Hkv
    out = torch.empty_like(x["q"])
    n_b = -(-S // 64)
    n_ret = int(x["is_retrieval"].sum())
    sel = torch.empty((n_ret, n_b, w.top_k + 2), dtype=torch.int32, device=dev)
    cnt = torch.empty((n_ret, n_b), dtype=torch.int32, device=dev)
    if dense:
        ws = torch.empty(rtp.dense_workspace_bytes(S, Hq, Hkv), dtype=torch.uint8,
                         device=dev)
        call = lambda: rtp.dense_attn_prefill(x["q"], x["k"], x["v"], ws=ws,
                                              out=out)
    elif full:
        wins = [w.window] * Hq
        ws = torch.empty(rtp.headwise_prefill_workspace_bytes(
            S, Hq, Hkv, x["is_retrieval"], "full", w.r, w.top_k),
            dtype=torch.uint8, device=dev)

        def call():
            return rtp.headwise_prefill(
                x["q"], x["k"], x["v"], x["is_retrieval"], wins, None, pk,
                w.top_k, retrieval="full", r=w.r, want_centroids=True, ws=ws,
                out=out)
    else:
        ws = torch.empty(rtp.prefill_workspace_bytes(S, Hq, Hkv,
                                                     x["is_retrieval"], w.r,
                                                     w.top_k),
                         dtype=torch.uint8, device=dev)

        def call():
            return rtp.hybrid_attn_prefill(
                x["q"], x["k"], x["v"], x["is_retrieval"], w.window, pq, pk,
                w.top_k, r=w.r, ws=ws, out=out)
    torch.cuda.synchronize()
    tag = ' dense' if dense else (' full-retrieval' if full else '')
    log(f"[bench] {w.name}{tag}: inputs ready in "
        f"{time.time() - t0:.1f}s, workspace {ws.numel() / 2**30:.2f} GiB")
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    with rtp.KernelTimer() as kt:
        t1 = time.perf_counter()
        for _ in range(steps):
            call()
        torch.cuda.synchronize()
        t2 = time.perf_counter()
    ms = (t2 - t1) * 1e3 / steps
    ks = kernel_stats(kt.records, steps)
    if dense:
        i = np.arange(S, dtype=np.int64)
        swa_pairs, ret_pairs = Hq * int((i + 1).sum()), 0
    elif full:
        # every head runs in the window kernel; retrieval heads causal-full
        i = np.arange(S, dtype=np.int64)
        swa_pairs, _ = prefill_pairs(S, Hq, x["is_retrieval"], w.window,
                                     np.zeros((0, n_b), dtype=np.int32))
        swa_pairs += n_ret * int((i + 1).sum())
        ret_pairs = 0
    else:
        # the selection of one more call, for exact pair counts
        _, _, s2, c2 = rtp.hybrid_attn_prefill(
            x["q"], x["k"], x["v"], x["is_retrieval"], w.window, pq, pk,
            w.top_k, r=w.r, ws=ws, out=out, want_sel=True)
        torch.cuda.synchronize()
        swa_pairs, ret_pairs = prefill_pairs(S, Hq, x["is_retrieval"],
                                             w.window, c2.cpu().numpy())
    flops = 4 * 128 * (swa_pairs + ret_pairs)
    win = ks.get("attn_window", {"ms_per_launch": float("nan")})
    spa = ks.get("attn_sparse", {"ms_per_launch": 0.0})
    att_ms = win["ms_per_launch"] + spa["ms_per_launch"]
    res = {
        "workload": w.name, "S": S, "ms_per_step": ms,
        "tokens_per_s": S / (ms / 1e3),
        "attn_pairs": {"window": swa_pairs, "retrieval": ret_pairs},
        "attn_flops": flops,
        "attn_ms": att_ms,
        "attn_tflops": flops / (att_ms / 1e3) / 1e12,
        "window_kernel_tflops": (4 * 128 * swa_pairs /
                                 (win["ms_per_launch"] / 1e3) / 1e12),
        "step_tflops": flops / (ms / 1e3) / 1e12,
        "kernels_ms_per_step": {k: round(v["ms_per_step"], 4)
                                for k, v in ks.items()},
    }
    if ret_pairs:
        res["sparse_kernel_tflops"] = (4 * 128 * ret_pairs /
                                       (spa["ms_per_launch"] / 1e3) / 1e12)
    res["attn_frac_bf16_peak"] = res["attn_tflops"] / PEAK_BF16_TFLOPS
    if not dense and not full and n_ret:
        # indexer figures (algorithmic). Scores: 2r flops per (query block,
        # candidate key), run as three bf16 MFMA products (hi.hi, hi.lo,
        # lo.hi), so the matrix cores execute 3x that. Projections: K of each
        # KV group with retrieval heads read once, the projected keys (64 B
        # per key per head) written once; Q of each retrieval head read once.
        cand_keys = 64 * sum(max(q - 1, 0) for q in range(n_b))
        G = Hq // Hkv
        n_grp = len({int(h) // G for h in x["retrieval_heads"]})
        sc = ks.get("score_select")
        if sc:
            alg = n_ret * cand_keys * 2 * w.r / (sc["ms_per_launch"] / 1e3)
            res["score_select_tflops_alg"] = alg / 1e12
            res["score_select_mfma_frac"] = 3 * alg / 1e12 / PEAK_BF16_TFLOPS
        pkk = ks.get("proj_keys")
        if pkk:
            byt = n_grp * S * 256 + n_ret * S * 64
            res["proj_keys_gbs_alg"] = byt / (pkk["ms_per_launch"] / 1e3) / 1e9
        pqm = ks.get("proj_qmeans")
        if pqm:
            byt = n_ret * S * 256
            res["proj_qmeans_gbs_alg"] = byt / (pqm["ms_per_launch"] / 1e3) / 1e9
        res["indexer_ms"] = sum(ks[k]["ms_per_launch"] for k in
                                ("proj_keys", "proj_qmeans", "score_select",
                                 "block_scores", "topk") if k in ks)
        bs = ks.get("block_scores")
        if bs:
            res["block_scores_tflops_alg"] = (n_ret * cand_keys * 2 * w.r /
                                              (bs["ms_per_launch"] / 1e3) / 1e12)
        res["workspace_gib"] = ws.numel() / 2**30
    if leg:
        res["hbm_counters"] = hbm_counters(leg, ks)
    del x, out, ws
    torch.cuda.empty_cache()
    return res


def gemm_reference(torch):
    """The vendor GEMM on the same device and clock: torch.matmul in bf16
    (hipBLASLt) at 16384 x 16384 x 8192. A practical matrix-core ceiling to
    read the attention kernels' fractions of the published peak against."""
    m, n, k = 16384, 16384, 8192
    a = torch.randn(m, k, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(k, n, dtype=torch.bfloat16, device="cuda")
    for _ in range(3):
        c = a @ b
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    del a, b, c
    torch.cuda.empty_cache()
    return {"gemm": f"torch.matmul bf16 {m}x{n}x{k}", "ms": ms,
            "tflops": 2 * m * n * k / (ms / 1e3) / 1e12}


def timed_steps(rtp, torch, call, steps, warmup):
    """Decode steps: the wall time per step from a loop without the
    per-kernel event timer (at a fraction of a millisecond per step, the
    events recorded around every kernel would add about a tenth), then the
    per-kernel times from a second, timed loop of as many steps."""
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t1) * 1e3 / steps
    with rtp.KernelTimer() as kt:
        for _ in range(steps):
            call()
        torch.cuda.synchronize()
    return ms, kernel_stats(kt.records, steps)


def bench_decode(rtp, torch, w, steps, warmup):
    from workloads import make_decode
    dev = "cuda"
    t0 = time.time()
    y = make_decode(w, device=dev)
    cl = torch.from_numpy(y["cache_len"]).to(dev)
    pq = torch.from_numpy(y["p_q"]).to(dev)
    pk = torch.from_numpy(y["p_k"]).to(dev)
    with rtp.KernelTimer() as kb:
        cent = rtp.build_centroids(y["k_cache"], cl, y["is_retrieval"], pk)
        torch.cuda.synchronize()
    B, Hq, Hkv, L = w.batch, w.Hq, w.Hkv, w.L
    ws = torch.empty(rtp.decode_workspace_bytes(B, L, Hq, Hkv,
                                                y["is_retrieval"], w.r,
                                                w.top_k, w.n_recent),
                     dtype=torch.uint8, device=dev)
    out = torch.empty_like(y["q"])

    def call(want_sel=False):
        return rtp.hybrid_attn_decode(y["q"], y["k_cache"], y["v_cache"], cl,
                                      y["is_retrieval"], w.window, pq, cent,
                                      w.top_k, n_recent=w.n_recent, ws=ws,
                                      out=out, want_sel=want_sel)
    torch.cuda.synchronize()
    log(f"[bench] {w.name}: inputs + centroids ready in {time.time() - t0:.1f}s")
    ms, ks = timed_steps(rtp, torch, call, steps, warmup)
    _, _, sel = call(want_sel=True)
    torch.cuda.synchronize()
    sel = sel.cpu().numpy()
    n_swa = int((y["is_retrieval"] == 0).sum())
    G = Hq // Hkv
    swa_groups = sum(1 for g in range(Hkv)
                     if any(not y["is_retrieval"][h]
                            for h in range(g * G, (g + 1) * G)))
    kv_row = 2 * 128 * 2  # K and V bytes per token
    win_bytes = B * swa_groups * min(w.window, L) * kv_row    # window passes
    ret_bytes = int((sel >= 0).sum()) * 64 * kv_row           # gathered blocks
    n_b = -(-L // 64)
    cen_bytes = B * sel.shape[1] * (n_b - w.n_recent - 1) * w.r * 4
    byt = win_bytes + ret_bytes + cen_bytes
    res = {
        "workload": w.name, "batch": B, "cache_len": L,
        "ms_per_step": ms, "tokens_per_s": B / (ms / 1e3),
        "bytes_per_step_alg": byt,
        "step_gbs_alg": byt / (ms / 1e3) / 1e9,
        "kernels_ms_per_step": {k: round(v["ms_per_step"], 4)
                                for k, v in ks.items()},
        "centroid_build_ms": kb.total("build_centroids"),
    }
    # streaming-head attention runs concurrently with the block choice and
    # the retrieval-head attention, so the kernel times overlap
    for name, part in (("dec_attn_window", win_bytes),
                       ("dec_attn_retrieval", ret_bytes)):
        if name in ks:
            res[name + "_gbs_alg"] = part / (ks[name]["ms_per_launch"] / 1e3) / 1e9
    res["step_frac_hbm"] = res["step_gbs_alg"] / PEAK_HBM_GBS
    res["hbm_counters"] = hbm_counters("decode", ks)
    del y, ws, out, cent
    torch.cuda.empty_cache()
    return res


PEAK_VALU_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12  # 32-bit VALU lane-ops/s
CLUSTER_ITERS = 2


def bench_cluster(rtp, torch, w, steps, warmup):
    """K-cache clustering (Lloyd steps seeded by the block centroids) and
    the clustered decode step on the decode workload."""
    from workloads import make_decode
    dev = "cuda"
    y = make_decode(w, device=dev)
    cl = torch.from_numpy(y["cache_len"]).to(dev)
    pq = torch.from_numpy(y["p_q"]).to(dev)
    pk = torch.from_numpy(y["p_k"]).to(dev)
    B, Hq, Hkv, L = w.batch, w.Hq, w.Hkv, w.L
    cent0 = rtp.build_centroids(y["k_cache"], cl, y["is_retrieval"], pk)
    cent = cent0.clone()
    cws = torch.empty(rtp.cluster_workspace_bytes(B, L, Hq, Hkv,
                                                  y["is_retrieval"], w.r),
                      dtype=torch.uint8, device=dev)
    tables = rtp.cluster_keys(y["k_cache"], cl, y["is_retrieval"], pk, cent,
                              iters=CLUSTER_ITERS, n_recent=w.n_recent, ws=cws)
    torch.cuda.synchronize()
    reps = 3
    with rtp.KernelTimer() as kc:
        t1 = time.perf_counter()
        for _ in range(reps):
            cent.copy_(cent0)
            rtp.cluster_keys(y["k_cache"], cl, y["is_retrieval"], pk, cent,
                             iters=CLUSTER_ITERS, n_recent=w.n_recent, ws=cws,
                             tables=tables)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
    cks = kernel_stats(kc.records, reps)
    cl_ms = sum(v["ms_total"] for k, v in cks.items()
                if k.startswith("cl_")) / reps
    ws = torch.empty(rtp.decode_clustered_workspace_bytes(
        B, L, Hq, Hkv, y["is_retrieval"], w.top_k, w.n_recent, w.r),
        dtype=torch.uint8, device=dev)
    out = torch.empty_like(y["q"])

    def call(want_sel=False):
        return rtp.hybrid_attn_decode_clustered(
            y["q"], y["k_cache"], y["v_cache"], cl, y["is_retrieval"],
            w.window, pq, cent, tables, w.top_k, n_recent=w.n_recent, ws=ws,
            out=out, want_sel=want_sel)
    ms, ks = timed_steps(rtp, torch, call, steps, warmup)
    _, _, sel = call(want_sel=True)
    torch.cuda.synchronize()
    sel = sel.cpu().numpy()
    m = tables[0].cpu().numpy()
    off = tables[1].cpu().numpy()
    n_b = -(-L // 64)
    kept = 0
    for b in range(B):
        for rho in range(sel.shape[1]):
            for c in sel[b, rho]:
                if c < 0:
                    continue
                c = int(c)
                kept += int(off[b, rho, c + 1] - off[b, rho, c]) \
                    if 1 <= c < m[b] else min(L, 64 * c + 64) - 64 * c
    G = Hq // Hkv
    swa_groups = sum(1 for g in range(Hkv)
                     if any(not y["is_retrieval"][h]
                            for h in range(g * G, (g + 1) * G)))
    kv_row = 2 * 128 * 2
    win_bytes = B * swa_groups * min(w.window, L) * kv_row
    ret_bytes = kept * kv_row
    cen_bytes = B * sel.shape[1] * (n_b - w.n_recent - 1) * w.r * 4
    byt = win_bytes + ret_bytes + cen_bytes
    # nearest-centroid search: (token, cluster) pairs of every (sequence,
    # head) per step, 3 VALU ops each (compare, two selects)
    C = m.astype(np.int64) - 1
    pairs = int(sel.shape[1] * (64 * C * C).sum())
    res = {
        "workload": w.name, "iters": CLUSTER_ITERS,
        "cluster_ms": cl_ms,
        "cluster_wall_ms": (t2 - t1) * 1e3 / reps,
        "cluster_kernels_ms": {k: round(v["ms_total"] / reps, 4)
                               for k, v in cks.items()},
        "assign_pairs_per_step": pairs,
        "decode_ms_per_step": ms, "decode_tokens_per_s": B / (ms / 1e3),
        "decode_kept_tokens": kept,
        "decode_bytes_per_step_alg": byt,
        "decode_step_gbs_alg": byt / (ms / 1e3) / 1e9,
        "decode_kernels_ms_per_step": {k: round(v["ms_per_step"], 4)
                                       for k, v in ks.items()},
    }
    if "cl_assign" in cks:
        t = cks["cl_assign"]["ms_per_launch"] / 1e3
        res["assign_valu_frac"] = 3 * pairs / t / 1e12 / PEAK_VALU_TOPS
    res["hbm_counters"] = hbm_counters("cluster", {**cks, **ks})
    del y, ws, out, cent, cent0, cws, tables
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------ CPU oracle
def cpu_baseline(w, ret_pairs_total, budget_s=15.0):
    """Time the oracle on a bounded sample of the workload and scale it to
    the whole layer by exact work counts (pairs, candidate keys)."""
    import torch
    import oracle
    from workloads import make_prefill, bf16_bits, draw_projections
    try:
        from threadpoolctl import threadpool_info
        blas = [p.get("num_threads") for p in threadpool_info()
                if p.get("user_api") == "blas"]
        cores = int(max(blas)) if blas else os.cpu_count()
    except Exception:
        cores = len(os.sched_getaffinity(0))
    x = make_prefill(w, device="cuda")
    S, B = w.S, 64
    n_b = -(-S // B)
    G = w.Hq // w.Hkv
    ret_heads = list(x["retrieval_heads"])
    swa_heads = [h for h in range(w.Hq) if not x["is_retrieval"][h]]
    h_r, h_s = ret_heads[0], swa_heads[0]
    g_r, g_s = h_r // G, h_s // G
    qr = oracle.bf16_to_f32(bf16_bits(x["q"][h_r]))
    kr = oracle.bf16_to_f32(bf16_bits(x["k"][g_r]))
    vr = oracle.bf16_to_f32(bf16_bits(x["v"][g_r]))
    qs = oracle.bf16_to_f32(bf16_bits(x["q"][h_s]))
    ks_ = oracle.bf16_to_f32(bf16_bits(x["k"][g_s]))
    vs = oracle.bf16_to_f32(bf16_bits(x["v"][g_s]))
    del x
    torch.cuda.empty_cache()
    scale = 1.0 / math.sqrt(128)
    rng = np.random.default_rng(1)
    t_start = time.perf_counter()
    # indexer of one retrieval head: projections in full
    t0 = time.perf_counter()
    p_q, p_k = draw_projections(len(ret_heads), w.r, 128, w.seed)
    khat = oracle.project_keys(kr, p_k[0])
    qbar = oracle.query_block_means(qr, p_q[0], B)
    t_proj = time.perf_counter() - t0
    # sampled selection rows and attention blocks, until the budget is used
    rows_done = cand_done = 0
    t_rows = 0.0
    ret_pairs = swa_pairs = 0
    t_ret = t_swa = 0.0
    i_blk = 0
    while time.perf_counter() - t_start < budget_s and i_blk < 20000:
        qb = int(rng.integers(2, n_b))
        t0 = time.perf_counter()
        sc = oracle.block_score_row(qbar[qb], khat, qb, B)
        sel, _, _ = oracle.select_row(sc, qb, w.top_k)
        t_rows += time.perf_counter() - t0
        rows_done += 1
        cand_done += qb - 1
        rows = np.arange(qb * B, min(S, (qb + 1) * B))
        t0 = time.perf_counter()
        union, mem = oracle.retrieval_block_keys(rows, sel, B, S)
        oracle.attend(qr[rows], kr[union], vr[union], mem, scale)
        t_ret += time.perf_counter() - t0
        ret_pairs += int(mem.sum())
        t0 = time.perf_counter()
        union, mem = oracle.swa_block_keys(rows, w.window)
        oracle.attend(qs[rows], ks_[union], vs[union], mem, scale)
        t_swa += time.perf_counter() - t0
        swa_pairs += int(mem.sum())
        i_blk += 1
    wall = time.perf_counter() - t_start
    # scale to the whole layer
    i = np.arange(S, dtype=np.int64)
    swa_total = int(np.minimum(i + 1, w.window).sum()) * len(swa_heads)
    cand_total = sum(max(q - 1, 0) for q in range(n_b))
    est = (len(ret_heads) * (t_proj + t_rows / max(cand_done, 1) * cand_total)
           + t_ret / max(ret_pairs, 1) * ret_pairs_total
           + t_swa / max(swa_pairs, 1) * swa_total)
    return {
        "value": S / est, "unit": "tokens/s", "cores": cores, "kind": "oracle",
        "sample": (f"{w.name}: indexer projections of 1 retrieval head, "
                   f"{rows_done} selection rows, {i_blk} query blocks of 1 "
                   f"retrieval and 1 window head ({wall:.1f}s of CPU work), "
                   f"scaled by exact pair / candidate counts to the whole "
                   f"layer (extrapolated {est:.0f}s)"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--only-main", action="store_true",
                    help="time the 128K prefill only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--leg", choices=["1m", "32k", "decode", "dense", "full",
                                      "dense1m", "cluster"],
                    help="run only this secondary leg and print its detail "
                         "(for profiling); no bench line")
    ap.add_argument("--copy-probe-gib", type=float, default=0.0,
                    help="after the timed legs, run a plain device copy of "
                         "this many GiB twice (calibrates HBM byte counters "
                         "under rocprofv3 --pmc)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU "
              "path (prefill would shard by KV group or by query positions, "
              "decode by sequence); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import long_context_sparse_head_amd as rtp
    from workloads import PREFILL_128K, PREFILL_1M, PREFILL_32K, DECODE_32x256K
    rtp.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    def copy_probe():
        # a plain device copy of known size, for calibrating byte counters
        n = int(args.copy_probe_gib * 2**30)
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: 2 x {n} bytes copied")
        del src, dst

    if args.leg:
        if args.leg == "decode":
            res = bench_decode(rtp, torch, DECODE_32x256K, args.steps,
                               args.warmup)
        elif args.leg == "cluster":
            res = bench_cluster(rtp, torch, DECODE_32x256K, args.steps,
                                args.warmup)
        else:
            w = {"1m": PREFILL_1M, "32k": PREFILL_32K,
                 "dense": PREFILL_128K, "full": PREFILL_128K,
                 "dense1m": PREFILL_1M}[args.leg]
            res = bench_prefill(rtp, torch, w, args.steps, args.warmup,
                                dense=args.leg in ("dense", "dense1m"),
                                full=args.leg == "full",
                                leg=args.leg if args.leg in ("1m", "32k")
                                else None)
        if args.copy_probe_gib > 0:
            copy_probe()
        print(json.dumps({"leg": args.leg, **res}), flush=True)
        return
    main = bench_prefill(rtp, torch, PREFILL_128K, args.steps, args.warmup,
                         leg="128k")
    log(f"[bench] 128K: {main['ms_per_step']:.3f} ms/step, "
        f"{main['tokens_per_s']:.3e} tok/s, window kernel "
        f"{main['window_kernel_tflops']:.0f} TF/s, sparse kernel "
        f"{main.get('sparse_kernel_tflops', 0):.0f} TF/s")
    extra = {}
    if not args.only_main:
        extra["prefill_1m"] = bench_prefill(rtp, torch, PREFILL_1M,
                                            max(2, args.steps // 4), 1,
                                            leg="1m")
        log(f"[bench] 1M: {extra['prefill_1m']['ms_per_step']:.1f} ms/step")
        extra["prefill_32k"] = bench_prefill(rtp, torch, PREFILL_32K,
                                             args.steps, args.warmup)
        log(f"[bench] 32K: {extra['prefill_32k']['ms_per_step']:.3f} ms/step")
        extra["decode"] = bench_decode(rtp, torch, DECODE_32x256K, args.steps,
                                       args.warmup)
        log(f"[bench] decode: {extra['decode']['ms_per_step']:.3f} ms/step")
        extra["cluster"] = bench_cluster(rtp, torch, DECODE_32x256K,
                                         args.steps, args.warmup)
        log(f"[bench] clustering ({CLUSTER_ITERS} steps): "
            f"{extra['cluster']['cluster_ms']:.2f} ms; clustered decode "
            f"{extra['cluster']['decode_ms_per_step']:.3f} ms/step")
        extra["dense_128k"] = bench_prefill(rtp, torch, PREFILL_128K,
                                            max(2, args.steps // 4), 1,
                                            dense=True)
        log(f"[bench] dense 128K: {extra['dense_128k']['ms_per_step']:.1f} "
            f"ms/step")
        extra["speedup_vs_dense_128k"] = (extra["dense_128k"]["ms_per_step"] /
                                          main["ms_per_step"])
        # the pages' comparison (full attention vs the hybrid, 32K to 1M):
        # the same dense engine at 32K and, for one step, at 1M
        extra["dense_32k"] = bench_prefill(rtp, torch, PREFILL_32K,
                                           max(2, args.steps // 2), 1,
                                           dense=True)
        extra["speedup_vs_dense_32k"] = (extra["dense_32k"]["ms_per_step"] /
                                         extra["prefill_32k"]["ms_per_step"])
        extra["dense_1m"] = bench_prefill(rtp, torch, PREFILL_1M, 1, 0,
                                          dense=True)
        extra["speedup_vs_dense_1m"] = (extra["dense_1m"]["ms_per_step"] /
                                        extra["prefill_1m"]["ms_per_step"])
        log(f"[bench] dense 32K: {extra['dense_32k']['ms_per_step']:.2f} ms, "
            f"dense 1M: {extra['dense_1m']['ms_per_step']:.0f} ms; hybrid "
            f"speedup {extra['speedup_vs_dense_32k']:.2f}x (32K), "
            f"{extra['speedup_vs_dense_128k']:.2f}x (128K), "
            f"{extra['speedup_vs_dense_1m']:.2f}x (1M)")
        extra["full_retrieval_128k"] = bench_prefill(
            rtp, torch, PREFILL_128K, max(2, args.steps // 2), 1, full=True)
        log(f"[bench] 128K with full retrieval heads: "
            f"{extra['full_retrieval_128k']['ms_per_step']:.2f} ms/step")
    gemm = gemm_reference(torch)
    gemm["window_kernel_frac"] = main["window_kernel_tflops"] / gemm["tflops"]
    log(f"[bench] vendor bf16 GEMM on this device: {gemm['tflops']:.0f} TF/s "
        f"(window kernel at {gemm['window_kernel_frac']:.2f} of it)")
    if args.copy_probe_gib > 0:
        copy_probe()
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(PREFILL_128K, main["attn_pairs"]["retrieval"],
                           args.cpu_seconds)
        log(f"[bench] cpu oracle: {cpu['value']:.1f} tok/s")
    w = PREFILL_128K
    line = {
        "metric": METRIC,
        "value": main["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "seq_len": w.S, "q_heads": w.Hq,
                   "kv_heads": w.Hkv, "head_dim": w.d,
                   "retrieval_heads": w.n_ret, "window": w.window,
                   "rank": w.r, "block": w.block, "top_k": w.top_k,
                   "needle_blocks": w.needles},
        "roofline": {"bound": "mfma", "kernel": "attn_window_kernel",
                     "achieved": main["window_kernel_tflops"],
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": main["window_kernel_tflops"] / PEAK_BF16_TFLOPS,
                     "traffic": measured_traffic()},
        "cpu_baseline": cpu,
        "detail": {"prefill_128k": main, "gemm_reference": gemm, **extra},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
