"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/rtp.h, and rejects bad arguments with the documented
status before touching the device."""
import ctypes
import os
import re

import numpy as np
import pytest

import long_context_sparse_head_amd as rtp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rtp.h")

pytestmark = pytest.mark.skipif(not os.path.exists(rtp.LIB_PATH),
                                reason="librtp.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rtp_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("rtp_indexer_select", "rtp_hybrid_attn_prefill",
              "rtp_hybrid_attn_decode", "rtp_build_centroids",
              "rtp_dense_attn_prefill", "rtp_prefill_workspace_bytes",
              "rtp_decode_workspace_bytes", "rtp_status_string",
              "rtp_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = rtp.load()
    for n in declared_functions():
        assert hasattr(lib, n), n
    # the binding's signature table covers the same set
    assert set(declared_functions()) == set(rtp._SIGS)


def test_status_strings_and_version():
    lib = rtp.load()
    assert lib.rtp_status_string(0) == b"ok"
    assert b"invalid" in lib.rtp_status_string(-1)
    assert b"unsupported" in lib.rtp_status_string(-2)
    assert b"workspace" in lib.rtp_status_string(-3)
    assert b"HIP" in lib.rtp_status_string(-4)
    assert b"gfx950" in lib.rtp_version()


def _mask(bits):
    m = np.array(bits, dtype=np.uint8)
    return m, m.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))


def test_workspace_queries():
    lib = rtp.load()
    m, mp = _mask([1, 0, 0, 0])
    S, n_b = 2048, 32
    got = lib.rtp_prefill_workspace_bytes(S, 4, 1, 128, mp, 16, 64, 8)
    al = lambda x: (x + 255) // 256 * 256
    # V^T and the indexer's scratch share one region (the indexer runs
    # first); then the selection and its counts. Indexer scratch of a short
    # sequence: projected keys (256 r bytes per block), two halves of the
    # query-block means, the score rows (lower triangle, fp32) and the work
    # counter.
    vt = al(1 * 128 * S * 2)
    idx = (al(n_b * 256 * 16) + 2 * al(n_b * 16 * 2) +
           al((n_b - 2) * (n_b - 1) // 2 * 4) + 256)
    want = max(vt, idx) + al(n_b * 10 * 4) + al(n_b * 4)
    assert got == want
    assert lib.rtp_prefill_workspace_bytes(S, 4, 1, 64, mp, 16, 64, 8) == 0
    assert lib.rtp_prefill_workspace_bytes(S, 4, 1, 128, mp, 16, 32, 8) == 0
    assert lib.rtp_prefill_workspace_bytes(S, 4, 1, 128, mp, 24, 64, 8) == 0
    assert lib.rtp_dense_workspace_bytes(S, 4, 1, 128) == al(128 * S * 2)
    assert lib.rtp_decode_workspace_bytes(2, 4096, 4, 1, 128, mp, 16, 64, 8,
                                          2) > 0


def _prefill(lib, mp, **kw):
    a = dict(q=1, k=1, v=1, S=128, Hq=4, Hkv=1, d=128, window=16, pq=1, pk=1,
             r=16, block=64, top_k=4, scale=0.0, sel_in=None, cnt_in=None,
             out=1, lse=None, sel_out=None, cnt_out=None, ws=None, wsb=0)
    a.update(kw)
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.rtp_hybrid_attn_prefill(
        P(a["q"]), P(a["k"]), P(a["v"]), a["S"], a["Hq"], a["Hkv"], a["d"],
        mp, a["window"], P(a["pq"]), P(a["pk"]), a["r"], a["block"],
        a["top_k"], a["scale"], P(a["sel_in"]), P(a["cnt_in"]), P(a["out"]),
        P(a["lse"]), P(a["sel_out"]), P(a["cnt_out"]), P(a["ws"]), a["wsb"],
        None)


def test_prefill_argument_validation_returns_codes():
    lib = rtp.load()
    m, mp = _mask([1, 0, 0, 0])
    assert _prefill(lib, mp, d=64) == -2
    assert _prefill(lib, mp, block=32) == -2
    assert _prefill(lib, mp, r=20) == -2
    assert _prefill(lib, mp, Hq=6, Hkv=4) == -1
    assert _prefill(lib, mp, S=-1) == -1
    assert _prefill(lib, mp, window=0) == -1
    assert _prefill(lib, mp, top_k=-1) == -1
    assert _prefill(lib, mp, q=None) == -1
    assert _prefill(lib, mp, pq=None) == -1
    assert _prefill(lib, mp, sel_in=8) == -1       # count missing
    assert _prefill(lib, mp, sel_out=8) == -1      # count missing
    assert _prefill(lib, mp) == -3                 # no workspace
    assert _prefill(lib, mp, ws=1 << 20 | 8, wsb=1 << 40) == -3  # misaligned
    assert b"workspace" in lib.rtp_last_error()
    assert _prefill(lib, mp, S=0) == 0             # empty: nothing to do
    assert _prefill(lib, mp, S=(1 << 24) - 63) == -2  # K past 4 GiB per head
    assert b"16777152" in lib.rtp_last_error()
    m2, mp2 = _mask([0] * 130)
    assert _prefill(lib, mp2, Hq=130, Hkv=130) == -2


def test_top_k_and_n_recent_are_capped_at_the_most_blocks():
    # 262 143 = (2^24 - 64) / 64 blocks: a larger budget could only overflow
    # the selection width (top_k + 2, top_k + 1 + n_recent), so it is refused
    lib = rtp.load()
    m, mp = _mask([1, 0, 0, 0])
    big = (1 << 31) - 2
    assert _prefill(lib, mp, top_k=262143) == -3   # valid, needs a workspace
    assert _prefill(lib, mp, top_k=262144) == -1
    assert _prefill(lib, mp, top_k=big) == -1
    assert b"262143" in lib.rtp_last_error()
    assert lib.rtp_prefill_workspace_bytes(128, 4, 1, 128, mp, 16, 64,
                                           big) == 0
    m1, mp1 = _mask([0, 1])
    assert lib.rtp_decode_workspace_bytes(2, 4096, 2, 1, 128, mp1, 16, 64, 8,
                                          262143) > 0
    assert lib.rtp_decode_workspace_bytes(2, 4096, 2, 1, 128, mp1, 16, 64, 8,
                                          262144) == 0
    assert lib.rtp_decode_workspace_bytes(2, 4096, 2, 1, 128, mp1, 16, 64,
                                          big, 2) == 0
    P = ctypes.c_void_p
    for top_k, n_recent in ((big, 2), (8, big)):
        st = lib.rtp_hybrid_attn_decode(P(1), P(1), P(1), P(1), 2, 4096, 2, 1,
                                        128, mp1, 64, P(1), P(1), 16, 64,
                                        top_k, n_recent, 0.0, P(1), None, None,
                                        None, 0, None)
        assert st == -1, (top_k, n_recent)


def _headwise(lib, mp, windows, **kw):
    a = dict(q=1, k=1, v=1, S=128, Hq=4, Hkv=1, d=128, mode=0, pq=1, pk=1,
             r=16, block=64, top_k=4, scale=0.0, sel_in=None, cnt_in=None,
             out=1, lse=None, sel_out=None, cnt_out=None, cent=None, ws=None,
             wsb=0)
    a.update(kw)
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    wp = None if windows is None else np.array(windows, dtype=np.int32)
    wptr = None if wp is None else wp.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    return lib.rtp_headwise_prefill(
        P(a["q"]), P(a["k"]), P(a["v"]), a["S"], a["Hq"], a["Hkv"], a["d"],
        mp, wptr, a["mode"], P(a["pq"]), P(a["pk"]), a["r"], a["block"],
        a["top_k"], a["scale"], P(a["sel_in"]), P(a["cnt_in"]), P(a["out"]),
        P(a["lse"]), P(a["sel_out"]), P(a["cnt_out"]), P(a["cent"]),
        P(a["ws"]), a["wsb"], None)


def test_long_sequence_workspace_has_no_score_rows():
    # past 4096 blocks the indexer keeps per-row candidate buffers instead of
    # score rows: at 1M tokens with 23 retrieval heads the whole prefill
    # workspace stays under 3 GiB (score rows alone would be 11.5 GiB)
    lib = rtp.load()
    hq = [1] * 23 + [0] * 9
    m, mp = _mask(hq)
    ws = lib.rtp_prefill_workspace_bytes(1 << 20, 32, 4, 128, mp, 16, 64, 256)
    assert 0 < ws < 3 * 2 ** 30, ws
    rows = 23 * (16384 - 2) * (16384 - 1) // 2 * 4
    assert ws < rows


def test_headwise_prefill_validation_and_workspace():
    lib = rtp.load()
    m, mp = _mask([1, 0, 0, 0])
    ok = [0, 16, 8192, 1]  # head 0 is a retrieval head: its entry is unused
    assert _headwise(lib, mp, None) == -1
    assert _headwise(lib, mp, [5, 16, 0, 1]) == -1          # a window of 0
    assert _headwise(lib, mp, ok, mode=2) == -1             # unknown mode
    assert _headwise(lib, mp, ok, mode=1, sel_in=8, cnt_in=8) == -1
    assert _headwise(lib, mp, ok, mode=1, sel_out=8, cnt_out=8) == -1
    assert _headwise(lib, mp, ok, mode=0, pq=None) == -1     # must select
    assert _headwise(lib, mp, ok, mode=1, pk=None, cent=8) == -1
    assert _headwise(lib, mp, ok, mode=1, pq=None) == -3     # fine, no ws
    assert _headwise(lib, mp, ok, d=64) == -2
    assert _headwise(lib, mp, ok, S=0) == 0
    S, n_b = 2048, 32
    sparse = lib.rtp_headwise_prefill_workspace_bytes(S, 4, 1, 128, mp, 0, 16,
                                                      64, 8)
    assert sparse == lib.rtp_prefill_workspace_bytes(S, 4, 1, 128, mp, 16, 64, 8)
    al = lambda x: (x + 255) // 256 * 256
    full = lib.rtp_headwise_prefill_workspace_bytes(S, 4, 1, 128, mp, 1, 16,
                                                    64, 8)
    assert full == al(128 * S * 2)  # V^T only: no selection, and the
    # centroid epilogue projects keys straight into the centroids
    assert lib.rtp_headwise_prefill_workspace_bytes(S, 4, 1, 128, mp, 3, 16,
                                                    64, 8) == 0


def test_decode_and_centroid_validation():
    lib = rtp.load()
    m, mp = _mask([0, 1])
    P = ctypes.c_void_p
    st = lib.rtp_hybrid_attn_decode(P(1), P(1), P(1), P(1), 2, 4096, 2, 1,
                                    128, mp, 0, P(1), P(1), 16, 64, 8, 2, 0.0,
                                    P(1), None, None, None, 0, None)
    assert st == -1  # window 0
    st = lib.rtp_hybrid_attn_decode(P(1), P(1), P(1), P(1), 2, 4096, 2, 1,
                                    128, mp, 64, None, P(1), 16, 64, 8, 2, 0.0,
                                    P(1), None, None, None, 0, None)
    assert st == -1  # p_q missing with a retrieval head
    st = lib.rtp_hybrid_attn_decode(P(1), P(1), P(1), P(1), 2, 4096, 2, 1,
                                    128, mp, 64, P(1), P(1), 16, 64, 8, 2, 0.0,
                                    P(1), None, None, None, 0, None)
    assert st == -3  # no workspace
    st = lib.rtp_build_centroids(P(1), P(1), 2, 4096, 2, 1, 128, mp, None, 16,
                                 64, P(1), None)
    assert st == -1
    st = lib.rtp_build_centroids(P(1), P(1), 2, 4096, 2, 1, 128, mp, P(1), 16,
                                 48, P(1), None)
    assert st == -2
    # append: retrieval head without p_k / centroids, bad d, bad block
    st = lib.rtp_decode_append(P(1), P(1), P(1), P(1), P(1), 2, 4096, 2, 1,
                               128, mp, None, 16, 64, None, None)
    assert st == -1
    st = lib.rtp_decode_append(P(1), P(1), P(1), P(1), P(1), 2, 4096, 2, 1,
                               64, mp, P(1), 16, 64, P(1), None)
    assert st == -2
    st = lib.rtp_decode_append(P(1), P(1), P(1), P(1), P(1), 2, 4096, 2, 1,
                               128, mp, P(1), 16, 32, P(1), None)
    assert st == -2
    st = lib.rtp_decode_append(None, P(1), P(1), P(1), P(1), 2, 4096, 2, 1,
                               128, mp, P(1), 16, 64, P(1), None)
    assert st == -1


def test_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(4, 64, 128, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        rtp.dense_attn_prefill(q, q[:1], q[:1])


def test_cluster_workspace_and_validation():
    lib = rtp.load()
    al = lambda x: (x + 255) // 256 * 256
    m, mp = _mask([0, 1, 1, 0])
    B, Lmax = 3, 64 * 50 + 7
    nb = Lmax // 64
    want = al(B * 2 * Lmax * 16 * 4) + al(B * 2 * Lmax * 4) + \
        al(B * 2 * 64 * nb * 4)
    assert lib.rtp_cluster_workspace_bytes(B, Lmax, 4, 2, 128, mp, 16, 64) \
        == want
    assert lib.rtp_cluster_workspace_bytes(B, Lmax, 4, 2, 128, mp, 80, 64) \
        == 0  # r > 64 is not clustered
    # the clustered decode adds the token lists to the decode workspace
    dec = lib.rtp_decode_workspace_bytes(B, Lmax, 4, 2, 128, mp, 16, 64, 8, 2)
    assert lib.rtp_decode_clustered_workspace_bytes(
        B, Lmax, 4, 2, 128, mp, 16, 64, 8, 2) == \
        dec + al(B * 2 * Lmax * 4) + al(B * 2 * 4)
    P = ctypes.c_void_p
    args = lambda **kw: dict(dict(kc=P(1), cl=P(1), r=16, nrec=2, it=1,
                                  tab=P(1), ws=P(256)), **kw)

    def call(a):
        return lib.rtp_cluster_keys(a["kc"], a["cl"], B, Lmax, 4, 2, 128, mp,
                                    P(1), a["r"], 64, a["nrec"], a["it"],
                                    P(1), a["tab"], a["tab"], a["tab"],
                                    a["ws"], 1 << 40, None)
    assert call(args(r=80)) == -2
    assert call(args(nrec=0)) == -1
    assert call(args(it=-1)) == -1
    assert call(args(kc=None)) == -1
    assert call(args(tab=None)) == -1
    assert call(args(ws=None)) == -3
    # clustered decode: tables missing with a retrieval head
    st = lib.rtp_hybrid_attn_decode_clustered(
        P(1), P(1), P(1), P(1), 2, 4096, 4, 2, 128, mp, 64, P(1), P(1), None,
        P(1), P(1), 16, 64, 8, 2, 0.0, P(1), None, None, P(256), 1 << 40,
        None)
    assert st == -1
    st = lib.rtp_hybrid_attn_decode_clustered(
        P(1), P(1), P(1), P(1), 2, 4096, 4, 2, 128, mp, 64, P(1), P(1), P(1),
        P(1), P(1), 16, 64, 8, 2, 0.0, P(1), None, None, None, 0, None)
    assert st == -3


def test_paged_validation():
    lib = rtp.load()
    m, mp = _mask([0, 1, 1, 0])
    P = ctypes.c_void_p
    # NULL block table, zero max_blocks, zero pages
    for table, mb, npg in ((None, 4, 8), (P(1), 0, 8), (P(1), 4, 0)):
        st = lib.rtp_hybrid_attn_decode_paged(
            P(1), P(1), P(1), table, mb, npg, P(1), 2, 4, 2, 128, mp, 64,
            P(1), P(1), 16, 64, 8, 2, 0.0, P(1), None, None, P(256), 1 << 40,
            None)
        assert st == -1
        assert lib.rtp_build_centroids_paged(
            P(1), table, mb, npg, P(1), 2, 4, 2, 128, mp, P(1), 16, 64, P(1),
            None) == -1
    # a valid table with no workspace: sized like the unpaged decode
    st = lib.rtp_hybrid_attn_decode_paged(
        P(1), P(1), P(1), P(1), 4, 8, P(1), 2, 4, 2, 128, mp, 64, P(1), P(1),
        16, 64, 8, 2, 0.0, P(1), None, None, None, 0, None)
    assert st == -3
