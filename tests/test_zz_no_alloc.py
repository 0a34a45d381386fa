"""The allocation-free decode entry point (rtp_hybrid_attn_decode_noalloc)
against the one that takes a workspace (rtp_hybrid_attn_decode), through the
C ABI.

Both run the same kernels, so every output must be bitwise equal (stricter
than the oracle tolerance the workspace entry point is held to). Two calls
in a row on one GPU share the library's scratch array, the second with a
smaller batch and shorter caches; a step that needs more scratch than the
array holds is refused before anything is launched.
"""
import ctypes

import numpy as np
import pytest
import torch

import long_context_sparse_head_amd as rtp
from workloads import DecodeWorkload, make_decode


def _case(B, lens, ret, window, top_k, seed):
    w = DecodeWorkload("noalloc", batch=B, L=max(lens), Hq=8, Hkv=2, d=128,
                       n_ret=len(ret), window=window, r=16, block=64,
                       top_k=top_k, seed=seed, retrieval_heads=tuple(ret))
    return make_decode(w, device="cuda", cache_len=lens)


@pytest.mark.gpu
def test_noalloc_decode_matches_workspace_entry_point(gpu_lib):
    cases = [(6, [5000, 4096, 777, 65, 4161, 1], (1, 6), 512, 8, 1),
             (3, [3000, 100, 2049], (0, 5), 256, 5, 2)]
    for B, lens, ret, window, top_k, seed in cases:
        print(f"[noalloc] B={B} lens={lens}", flush=True)
        y = _case(B, lens, ret, window, top_k, seed)
        cl = torch.from_numpy(y["cache_len"]).cuda()
        pq = torch.from_numpy(y["p_q"]).cuda()
        pk = torch.from_numpy(y["p_k"]).cuda()
        cent = gpu_lib.build_centroids(y["k_cache"], cl, y["is_retrieval"], pk)
        ref_out, ref_lse, ref_sel = gpu_lib.hybrid_attn_decode(
            y["q"], y["k_cache"], y["v_cache"], cl, y["is_retrieval"], window,
            pq, cent, top_k, n_recent=2, want_lse=True, want_sel=True)
        out = torch.empty_like(y["q"])
        lse = torch.empty_like(ref_lse)
        sel = torch.empty_like(ref_sel)
        gpu_lib.hybrid_attn_decode_noalloc(
            y["q"], y["k_cache"], y["v_cache"], cl, y["is_retrieval"], window,
            pq, cent, top_k, n_recent=2, out=out, lse=lse, sel=sel)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out)
        assert torch.equal(lse, ref_lse)
        assert torch.equal(sel, ref_sel)


def test_noalloc_rejects_steps_beyond_its_scratch():
    # 1024 sequences x 32 heads x 8 splits of 128 fp32 partial outputs alone
    # are 128 MiB: refused with RTP_EWORKSPACE before any pointer is used
    lib = rtp.load()
    m = np.zeros(32, dtype=np.uint8)
    m[[3, 9]] = 1
    mp = m.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))
    need = lib.rtp_decode_workspace_bytes(1024, 4096, 32, 4, 128, mp, 16, 64,
                                          8, 2)
    assert need > rtp.NOALLOC_SCRATCH_BYTES
    st = lib.rtp_hybrid_attn_decode_noalloc(
        1, 1, 1, 1, 1024, 4096, 32, 4, 128, mp, 64, 1, 1, 16, 64, 8, 2, 0.0,
        1, None, None, None)
    assert st == -3
    msg = lib.rtp_last_error()
    assert str(need).encode() in msg and b"noalloc" in msg
    # a step that fits is not refused for its size (no GPU here: it then
    # fails on the device lookup or launch, never with RTP_EWORKSPACE)
    small = lib.rtp_decode_workspace_bytes(2, 4096, 32, 4, 128, mp, 16, 64, 8,
                                           2)
    assert small <= rtp.NOALLOC_SCRATCH_BYTES
