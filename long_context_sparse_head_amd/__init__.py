"""Headwise hybrid attention on MI355X (gfx950): Python binding of librtp.so.

Streaming heads run causal sliding-window attention; retrieval heads use an
r = 16 low-rank indexer to keep a few 64-token key blocks (sink, diagonal and
the top-k by block score) and run exact softmax attention on them; decode
scores per-block key centroids instead. All computation runs in the HIP
library; this module only checks tensors and passes pointers, sizes and the
current HIP stream through the C ABI declared in include/rtp.h. PyTorch is
used for device memory and streams only.

The library must be built (``python -m long_context_sparse_head_amd.build``);
every call raises if it is missing. There is no fallback.

A layer, end to end (bf16 tensors on the GPU; ``is_retrieval`` a host
sequence of 0/1 per query head; ``p_q``, ``p_k`` fp32 [n_ret, r, 128])::

    import long_context_sparse_head_amd as rtp
    # prefill: q [Hq,S,128], k and v [Hkv,S,128]
    out = rtp.hybrid_attn_prefill(q, k, v, is_retrieval, 8192, p_q, p_k,
                                  top_k=64)
    # decode cache [B,Hkv,Lmax,128] holding the prompt; lengths int32 [B]
    cent = rtp.build_centroids(k_cache, cache_len, is_retrieval, p_k)
    for _ in range(steps):
        rtp.decode_append(k_cache, v_cache, cache_len, k_new, v_new,
                          is_retrieval, p_k, cent)   # k_new [B,Hkv,128]
        o = rtp.hybrid_attn_decode(q_t, k_cache, v_cache, cache_len,
                                   is_retrieval, 8192, p_q, cent, top_k=64)
    # or cluster the keys first and decode over the clusters
    tables = rtp.cluster_keys(k_cache, cache_len, is_retrieval, p_k, cent,
                              iters=2)
    o = rtp.hybrid_attn_decode_clustered(q_t, k_cache, v_cache, cache_len,
                                         is_retrieval, 8192, p_q, cent,
                                         tables, top_k=64)

Each call has a ``*_workspace_bytes`` companion; passing ``ws=`` (a
uint8 tensor of that size) avoids an allocation per call. Paged caches go
through :class:`PagedCache` and the ``*_paged`` calls.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

__all__ = [
    "load", "LIB_PATH", "RtpError", "prefill_workspace_bytes",
    "headwise_prefill_workspace_bytes",
    "dense_workspace_bytes", "decode_workspace_bytes", "indexer_select",
    "hybrid_attn_prefill", "headwise_prefill", "dense_attn_prefill",
    "build_centroids",
    "hybrid_attn_decode", "hybrid_attn_decode_noalloc", "decode_append",
    "version", "KernelTimer", "NOALLOC_SCRATCH_BYTES",
    "cluster_workspace_bytes", "cluster_keys",
    "decode_clustered_workspace_bytes", "hybrid_attn_decode_clustered",
    "PagedCache", "build_centroids_paged", "decode_append_paged",
    "hybrid_attn_decode_paged", "cluster_keys_paged",
    "hybrid_attn_decode_clustered_paged",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib",
                        "librtp.so")
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t
_U8P = ctypes.POINTER(ctypes.c_uint8)
_I32P = ctypes.POINTER(ctypes.c_int32)

_SIGS = {
    "rtp_status_string": (ctypes.c_char_p, [_I]),
    "rtp_last_error": (ctypes.c_char_p, []),
    "rtp_version": (ctypes.c_char_p, []),
    "rtp_profile": (_I, [_I]),
    "rtp_profile_read": (_I, [ctypes.POINTER(ctypes.c_char_p),
                              ctypes.POINTER(ctypes.c_float), _I]),
    "rtp_prefill_workspace_bytes": (_Z, [_I, _I, _I, _I, _U8P, _I, _I, _I]),
    "rtp_dense_workspace_bytes": (_Z, [_I, _I, _I, _I]),
    "rtp_decode_workspace_bytes": (_Z, [_I, _I, _I, _I, _I, _U8P, _I, _I, _I,
                                        _I]),
    "rtp_indexer_select": (_I, [_P, _P, _I, _I, _I, _I, _U8P, _P, _P, _I, _I,
                                _I, _P, _P, _P, _P, _P, _Z, _P]),
    "rtp_hybrid_attn_prefill": (_I, [_P, _P, _P, _I, _I, _I, _I, _U8P, _I, _P,
                                     _P, _I, _I, _I, _F, _P, _P, _P, _P, _P,
                                     _P, _P, _Z, _P]),
    "rtp_dense_attn_prefill": (_I, [_P, _P, _P, _I, _I, _I, _I, _F, _P, _P,
                                    _P, _Z, _P]),
    "rtp_headwise_prefill_workspace_bytes": (_Z, [_I, _I, _I, _I, _U8P, _I,
                                                  _I, _I, _I]),
    "rtp_headwise_prefill": (_I, [_P, _P, _P, _I, _I, _I, _I, _U8P, _I32P, _I,
                                  _P, _P, _I, _I, _I, _F, _P, _P, _P, _P, _P,
                                  _P, _P, _P, _Z, _P]),
    "rtp_build_centroids": (_I, [_P, _P, _I, _I, _I, _I, _I, _U8P, _P, _I, _I,
                                 _P, _P]),
    "rtp_decode_append": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _U8P,
                               _P, _I, _I, _P, _P]),
    "rtp_hybrid_attn_decode": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _U8P,
                                    _I, _P, _P, _I, _I, _I, _I, _F, _P, _P, _P,
                                    _P, _Z, _P]),
    "rtp_hybrid_attn_decode_noalloc": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I,
                                            _U8P, _I, _P, _P, _I, _I, _I, _I,
                                            _F, _P, _P, _P, _P]),
    "rtp_cluster_workspace_bytes": (_Z, [_I, _I, _I, _I, _I, _U8P, _I, _I]),
    "rtp_cluster_keys": (_I, [_P, _P, _I, _I, _I, _I, _I, _U8P, _P, _I, _I,
                              _I, _I, _P, _P, _P, _P, _P, _Z, _P]),
    "rtp_decode_clustered_workspace_bytes": (_Z, [_I, _I, _I, _I, _I, _U8P,
                                                  _I, _I, _I, _I]),
    "rtp_hybrid_attn_decode_clustered": (_I, [_P, _P, _P, _P, _I, _I, _I, _I,
                                              _I, _U8P, _I, _P, _P, _P, _P, _P,
                                              _I, _I, _I, _I, _F, _P, _P, _P,
                                              _P, _Z, _P]),
    "rtp_build_centroids_paged": (_I, [_P, _P, _I, _I, _P, _I, _I, _I, _I,
                                       _U8P, _P, _I, _I, _P, _P]),
    "rtp_decode_append_paged": (_I, [_P, _P, _P, _I, _I, _P, _P, _P, _I, _I,
                                     _I, _I, _U8P, _P, _I, _I, _P, _P]),
    "rtp_hybrid_attn_decode_paged": (_I, [_P, _P, _P, _P, _I, _I, _P, _I, _I,
                                          _I, _I, _U8P, _I, _P, _P, _I, _I,
                                          _I, _I, _F, _P, _P, _P, _P, _Z, _P]),
    "rtp_cluster_keys_paged": (_I, [_P, _P, _I, _I, _P, _I, _I, _I, _I, _U8P,
                                    _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _Z,
                                    _P]),
    "rtp_hybrid_attn_decode_clustered_paged": (_I, [
        _P, _P, _P, _P, _I, _I, _P, _I, _I, _I, _I, _U8P, _I, _P, _P, _P, _P,
        _P, _I, _I, _I, _I, _F, _P, _P, _P, _P, _Z, _P]),
}


class RtpError(RuntimeError):
    pass


def load():
    """Load librtp.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RtpError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m long_context_sparse_head_amd.build`")
        _warn_if_stale()
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _warn_if_stale():
    import warnings
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    try:
        newest = max(os.path.getmtime(os.path.join(src, f))
                     for f in os.listdir(src))
    except (OSError, ValueError):
        return
    if newest > os.path.getmtime(LIB_PATH):
        warnings.warn(f"{LIB_PATH} is older than its sources in {src}; "
                      "rebuild with `python -m long_context_sparse_head_amd.build`")


def version() -> str:
    return load().rtp_version().decode()


class KernelTimer:
    """Per-kernel HIP-event timing of library calls made inside the block.

    with KernelTimer() as kt: ...; then kt.records = [(name, ms), ...]."""

    def __enter__(self):
        load().rtp_profile(1)
        self.records = []
        return self

    def __exit__(self, *exc):
        lib = load()
        cap = 1 << 14
        names = (ctypes.c_char_p * cap)()
        ms = (ctypes.c_float * cap)()
        n = lib.rtp_profile_read(names, ms, cap)
        lib.rtp_profile(0)
        if n < 0:
            _check(n, "rtp_profile_read")
        self.records = [(names[i].decode(), float(ms[i])) for i in range(n)]
        return False

    def total(self, name: str) -> float:
        return sum(t for k, t in self.records if k == name)

    def count(self, name: str) -> int:
        return sum(1 for k, _ in self.records if k == name)


def _check(status: int, what: str):
    if status != 0:
        lib = load()
        raise RtpError(f"{what}: {lib.rtp_status_string(status).decode()}: "
                       f"{lib.rtp_last_error().decode()}")


def _mask(is_retrieval, Hq: int):
    m = np.ascontiguousarray(np.asarray(is_retrieval, dtype=np.uint8))
    if m.shape != (Hq,):
        raise ValueError(f"is_retrieval must have shape ({Hq},)")
    return m, m.ctypes.data_as(_U8P)


def _dev(t: Optional[torch.Tensor], dtype, name: str, shape=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA/HIP tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, "
                         f"got {tuple(t.shape)}")
    return t


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]):
    if ws is not None:
        _dev(ws, torch.uint8, "ws")
        if ws.numel() < nbytes:
            raise ValueError(f"workspace needs {nbytes} bytes")
        return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def prefill_workspace_bytes(S: int, Hq: int, Hkv: int, is_retrieval,
                            r: int = 16, top_k: int = 64, d: int = 128,
                            block: int = 64) -> int:
    m, mp = _mask(is_retrieval, Hq)
    return int(load().rtp_prefill_workspace_bytes(S, Hq, Hkv, d, mp, r, block,
                                                  top_k))


def headwise_prefill_workspace_bytes(S: int, Hq: int, Hkv: int, is_retrieval,
                                     retrieval: str = "sparse", r: int = 16,
                                     top_k: int = 64, d: int = 128,
                                     block: int = 64) -> int:
    m, mp = _mask(is_retrieval, Hq)
    return int(load().rtp_headwise_prefill_workspace_bytes(
        S, Hq, Hkv, d, mp, RETRIEVAL_MODES[retrieval], r, block, top_k))


def dense_workspace_bytes(S: int, Hq: int, Hkv: int, d: int = 128) -> int:
    return int(load().rtp_dense_workspace_bytes(S, Hq, Hkv, d))


def decode_workspace_bytes(B: int, Lmax: int, Hq: int, Hkv: int, is_retrieval,
                           r: int = 16, top_k: int = 64, n_recent: int = 2,
                           d: int = 128, block: int = 64) -> int:
    m, mp = _mask(is_retrieval, Hq)
    return int(load().rtp_decode_workspace_bytes(B, Lmax, Hq, Hkv, d, mp, r,
                                                 block, top_k, n_recent))


def _proj(p, n_ret, r, d, name):
    if n_ret == 0:
        return None
    return _dev(p, torch.float32, name, (n_ret, r, d))


def indexer_select(q, k, is_retrieval, p_q, p_k, top_k: int, r: int = 16,
                   block: int = 64, kth: bool = False,
                   centroids: bool = False, ws=None):
    """Returns (sel [n_ret,n_b,top_k+2], sel_count [n_ret,n_b],
    kth [n_ret,n_b,2] or None, centroids [n_ret,n_b,r] or None)."""
    lib = load()
    Hq, S, d = q.shape
    Hkv = k.shape[0]
    _dev(q, torch.bfloat16, "q", (Hq, S, d))
    _dev(k, torch.bfloat16, "k", (Hkv, S, d))
    m, mp = _mask(is_retrieval, Hq)
    n_ret = int(m.astype(bool).sum())
    _proj(p_q, n_ret, r, d, "p_q")
    _proj(p_k, n_ret, r, d, "p_k")
    n_b = -(-S // block)
    dev = q.device
    sel = torch.full((n_ret, n_b, top_k + 2), -1, dtype=torch.int32, device=dev)
    cnt = torch.zeros((n_ret, n_b), dtype=torch.int32, device=dev)
    kt = torch.empty((n_ret, n_b, 2), dtype=torch.float32, device=dev) \
        if kth else None
    ce = torch.empty((n_ret, n_b, r), dtype=torch.float32, device=dev) \
        if centroids else None
    nb = lib.rtp_prefill_workspace_bytes(S, Hq, Hkv, d, mp, r, block, top_k)
    w = _workspace(nb, dev, ws)
    _check(lib.rtp_indexer_select(
        _ptr(q), _ptr(k), S, Hq, Hkv, d, mp, _ptr(p_q), _ptr(p_k), r, block,
        top_k, _ptr(sel), _ptr(cnt), _ptr(kt), _ptr(ce), _ptr(w), w.numel(),
        _stream(dev)), "rtp_indexer_select")
    return sel, cnt, kt, ce


def hybrid_attn_prefill(q, k, v, is_retrieval, window: int, p_q, p_k,
                        top_k: int, r: int = 16, block: int = 64,
                        scale: float = 0.0, sel=None, sel_count=None,
                        want_lse: bool = False, want_sel: bool = False,
                        ws=None, out=None):
    """One layer of hybrid prefill. Returns out, or a tuple
    (out, lse, sel, sel_count) with None for the parts not asked for."""
    lib = load()
    Hq, S, d = q.shape
    Hkv = k.shape[0]
    _dev(q, torch.bfloat16, "q", (Hq, S, d))
    _dev(k, torch.bfloat16, "k", (Hkv, S, d))
    _dev(v, torch.bfloat16, "v", (Hkv, S, d))
    m, mp = _mask(is_retrieval, Hq)
    n_ret = int(m.astype(bool).sum())
    n_b = -(-S // block)
    dev = q.device
    if sel is not None:
        _dev(sel, torch.int32, "sel", (n_ret, n_b, top_k + 2))
        _dev(sel_count, torch.int32, "sel_count", (n_ret, n_b))
    else:
        _proj(p_q, n_ret, r, d, "p_q")
        _proj(p_k, n_ret, r, d, "p_k")
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev(out, torch.bfloat16, "out", (Hq, S, d))
    lse = torch.empty((Hq, S), dtype=torch.float32, device=dev) \
        if want_lse else None
    so = co = None
    if want_sel:
        so = torch.full((n_ret, n_b, top_k + 2), -1, dtype=torch.int32,
                        device=dev)
        co = torch.zeros((n_ret, n_b), dtype=torch.int32, device=dev)
    nb = lib.rtp_prefill_workspace_bytes(S, Hq, Hkv, d, mp, r, block, top_k)
    w = _workspace(nb, dev, ws)
    _check(lib.rtp_hybrid_attn_prefill(
        _ptr(q), _ptr(k), _ptr(v), S, Hq, Hkv, d, mp, int(window), _ptr(p_q),
        _ptr(p_k), r, block, top_k, float(scale), _ptr(sel), _ptr(sel_count),
        _ptr(out), _ptr(lse), _ptr(so), _ptr(co), _ptr(w), w.numel(),
        _stream(dev)), "rtp_hybrid_attn_prefill")
    if want_lse or want_sel:
        return out, lse, so, co
    return out


RETRIEVAL_MODES = {"sparse": 0, "full": 1}


def headwise_prefill(q, k, v, is_retrieval, windows, p_q, p_k, top_k: int,
                     retrieval: str = "sparse", r: int = 16, block: int = 64,
                     scale: float = 0.0, sel=None, sel_count=None,
                     want_lse: bool = False, want_sel: bool = False,
                     want_centroids: bool = False, ws=None, out=None):
    """Prefill with a window per head (host int sequence of length Hq) and
    retrieval heads either "sparse" (indexer selection) or "full" (causal
    full attention). Returns out, or a tuple (out, lse, sel, sel_count,
    centroids) with None for the parts not asked for."""
    lib = load()
    Hq, S, d = q.shape
    Hkv = k.shape[0]
    _dev(q, torch.bfloat16, "q", (Hq, S, d))
    _dev(k, torch.bfloat16, "k", (Hkv, S, d))
    _dev(v, torch.bfloat16, "v", (Hkv, S, d))
    if retrieval not in RETRIEVAL_MODES:
        raise ValueError(f"retrieval must be one of {sorted(RETRIEVAL_MODES)}")
    mode = RETRIEVAL_MODES[retrieval]
    m, mp = _mask(is_retrieval, Hq)
    win = np.ascontiguousarray(np.asarray(windows, dtype=np.int32))
    if win.shape != (Hq,):
        raise ValueError(f"windows must have {Hq} entries")
    wp = win.ctypes.data_as(_I32P)
    n_ret = int(m.astype(bool).sum())
    n_b = -(-S // block)
    dev = q.device
    if sel is not None:
        _dev(sel, torch.int32, "sel", (n_ret, n_b, top_k + 2))
        _dev(sel_count, torch.int32, "sel_count", (n_ret, n_b))
    elif mode == 0:
        _proj(p_q, n_ret, r, d, "p_q")
    if (mode == 0 and sel is None) or want_centroids:
        _proj(p_k, n_ret, r, d, "p_k")
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev(out, torch.bfloat16, "out", (Hq, S, d))
    lse = torch.empty((Hq, S), dtype=torch.float32, device=dev) \
        if want_lse else None
    so = co = None
    if want_sel:
        so = torch.full((n_ret, n_b, top_k + 2), -1, dtype=torch.int32,
                        device=dev)
        co = torch.zeros((n_ret, n_b), dtype=torch.int32, device=dev)
    cent = torch.zeros((n_ret, n_b, r), dtype=torch.float32, device=dev) \
        if want_centroids else None
    nb = lib.rtp_headwise_prefill_workspace_bytes(S, Hq, Hkv, d, mp, mode, r,
                                                  block, top_k)
    w = _workspace(nb, dev, ws)
    _check(lib.rtp_headwise_prefill(
        _ptr(q), _ptr(k), _ptr(v), S, Hq, Hkv, d, mp, wp, mode, _ptr(p_q),
        _ptr(p_k), r, block, top_k, float(scale), _ptr(sel), _ptr(sel_count),
        _ptr(out), _ptr(lse), _ptr(so), _ptr(co), _ptr(cent), _ptr(w),
        w.numel(), _stream(dev)), "rtp_headwise_prefill")
    if want_lse or want_sel or want_centroids:
        return out, lse, so, co, cent
    return out


def dense_attn_prefill(q, k, v, scale: float = 0.0, want_lse: bool = False,
                       ws=None, out=None):
    """Dense causal attention on the same tile engine (baseline)."""
    lib = load()
    Hq, S, d = q.shape
    Hkv = k.shape[0]
    _dev(q, torch.bfloat16, "q", (Hq, S, d))
    _dev(k, torch.bfloat16, "k", (Hkv, S, d))
    _dev(v, torch.bfloat16, "v", (Hkv, S, d))
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    lse = torch.empty((Hq, S), dtype=torch.float32, device=dev) \
        if want_lse else None
    w = _workspace(lib.rtp_dense_workspace_bytes(S, Hq, Hkv, d), dev, ws)
    _check(lib.rtp_dense_attn_prefill(
        _ptr(q), _ptr(k), _ptr(v), S, Hq, Hkv, d, float(scale), _ptr(out),
        _ptr(lse), _ptr(w), w.numel(), _stream(dev)), "rtp_dense_attn_prefill")
    return (out, lse) if want_lse else out


def build_centroids(k_cache, cache_len, is_retrieval, p_k, r: int = 16,
                    block: int = 64, out=None):
    """Per-block key centroids [B,n_ret,Lmax/block,r] (full blocks only)."""
    lib = load()
    B, Hkv, Lmax, d = k_cache.shape
    Hq = len(is_retrieval)
    _dev(k_cache, torch.bfloat16, "k_cache")
    _dev(cache_len, torch.int32, "cache_len", (B,))
    m, mp = _mask(is_retrieval, Hq)
    n_ret = int(m.astype(bool).sum())
    _proj(p_k, n_ret, r, d, "p_k")
    if out is None:
        out = torch.zeros((B, n_ret, Lmax // block, r), dtype=torch.float32,
                          device=k_cache.device)
    _check(lib.rtp_build_centroids(
        _ptr(k_cache), _ptr(cache_len), B, Lmax, Hq, Hkv, d, mp, _ptr(p_k), r,
        block, _ptr(out), _stream(k_cache.device)), "rtp_build_centroids")
    return out


def decode_append(k_cache, v_cache, cache_len, k_new, v_new, is_retrieval,
                  p_k=None, centroids=None, r: int = 16, block: int = 64):
    """Appends k_new/v_new [B,Hkv,d] at cache_len (in place), adds the
    centroid of each block the token completes, increments cache_len."""
    lib = load()
    B, Hkv, Lmax, d = k_cache.shape
    Hq = len(is_retrieval)
    _dev(k_cache, torch.bfloat16, "k_cache")
    _dev(v_cache, torch.bfloat16, "v_cache", (B, Hkv, Lmax, d))
    _dev(cache_len, torch.int32, "cache_len", (B,))
    _dev(k_new, torch.bfloat16, "k_new", (B, Hkv, d))
    _dev(v_new, torch.bfloat16, "v_new", (B, Hkv, d))
    m, mp = _mask(is_retrieval, Hq)
    n_ret = int(m.astype(bool).sum())
    if n_ret:
        _proj(p_k, n_ret, r, d, "p_k")
        _dev(centroids, torch.float32, "centroids",
             (B, n_ret, Lmax // block, r))
    _check(lib.rtp_decode_append(
        _ptr(k_cache), _ptr(v_cache), _ptr(cache_len), _ptr(k_new),
        _ptr(v_new), B, Lmax, Hq, Hkv, d, mp,
        _ptr(p_k) if n_ret else None, r, block,
        _ptr(centroids) if n_ret else None, _stream(k_cache.device)),
        "rtp_decode_append")


def hybrid_attn_decode(q, k_cache, v_cache, cache_len, is_retrieval,
                       window: int, p_q, centroids, top_k: int,
                       n_recent: int = 2, r: int = 16, block: int = 64,
                       scale: float = 0.0, want_lse: bool = False,
                       want_sel: bool = False, ws=None, out=None):
    """One decode step. Returns out, or (out, lse, sel) when asked."""
    lib = load()
    B, Hq, d = q.shape
    _, Hkv, Lmax, _ = k_cache.shape
    _dev(q, torch.bfloat16, "q", (B, Hq, d))
    _dev(k_cache, torch.bfloat16, "k_cache", (B, Hkv, Lmax, d))
    _dev(v_cache, torch.bfloat16, "v_cache", (B, Hkv, Lmax, d))
    _dev(cache_len, torch.int32, "cache_len", (B,))
    m, mp = _mask(is_retrieval, Hq)
    n_ret = int(m.astype(bool).sum())
    if n_ret:
        _proj(p_q, n_ret, r, d, "p_q")
        _dev(centroids, torch.float32, "centroids",
             (B, n_ret, Lmax // block, r))
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) \
        if want_lse else None
    so = torch.full((B, n_ret, top_k + 1 + n_recent), -1, dtype=torch.int32,
                    device=dev) if want_sel else None
    nb = lib.rtp_decode_workspace_bytes(B, Lmax, Hq, Hkv, d, mp, r, block,
                                        top_k, n_recent)
    w = _workspace(nb, dev, ws)
    _check(lib.rtp_hybrid_attn_decode(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_len), B, Lmax, Hq,
        Hkv, d, mp, int(window), _ptr(p_q), _ptr(centroids), r, block, top_k,
        n_recent, float(scale), _ptr(out), _ptr(lse), _ptr(so), _ptr(w),
        w.numel(), _stream(dev)), "rtp_hybrid_attn_decode")
    if want_lse or want_sel:
        return out, lse, so
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20  # RTP_NOALLOC_SCRATCH_BYTES


def hybrid_attn_decode_noalloc(q, k_cache, v_cache, cache_len, is_retrieval,
                               window: int, p_q, centroids, top_k: int,
                               n_recent: int = 2, r: int = 16, block: int = 64,
                               scale: float = 0.0, out=None, lse=None,
                               sel=None):
    """hybrid_attn_decode through rtp_hybrid_attn_decode_noalloc: the
    library's own static scratch, nothing allocated by the call. Outputs
    (out, and optionally lse [B,Hq] fp32 and sel [B,n_ret,top_k+1+n_recent]
    int32) are caller tensors; out is created only when not given."""
    lib = load()
    B, Hq, d = q.shape
    _, Hkv, Lmax, _ = k_cache.shape
    _dev(q, torch.bfloat16, "q", (B, Hq, d))
    _dev(k_cache, torch.bfloat16, "k_cache", (B, Hkv, Lmax, d))
    _dev(v_cache, torch.bfloat16, "v_cache", (B, Hkv, Lmax, d))
    _dev(cache_len, torch.int32, "cache_len", (B,))
    m, mp = _mask(is_retrieval, Hq)
    n_ret = int(m.astype(bool).sum())
    if n_ret:
        _proj(p_q, n_ret, r, d, "p_q")
        _dev(centroids, torch.float32, "centroids",
             (B, n_ret, Lmax // block, r))
    if out is None:
        out = torch.empty_like(q)
    _dev(out, torch.bfloat16, "out", (B, Hq, d))
    if lse is not None:
        _dev(lse, torch.float32, "lse", (B, Hq))
    if sel is not None:
        _dev(sel, torch.int32, "sel", (B, n_ret, top_k + 1 + n_recent))
    _check(lib.rtp_hybrid_attn_decode_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_len), B, Lmax, Hq,
        Hkv, d, mp, int(window), _ptr(p_q), _ptr(centroids), r, block, top_k,
        n_recent, float(scale), _ptr(out), _ptr(lse), _ptr(sel),
        _stream(q.device)), "rtp_hybrid_attn_decode_noalloc")
    return out


def cluster_workspace_bytes(B: int, Lmax: int, Hq: int, Hkv: int,
                            is_retrieval, r: int = 16, d: int = 128,
                            block: int = 64) -> int:
    _, mp = _mask(is_retrieval, Hq)
    return int(load().rtp_cluster_workspace_bytes(B, Lmax, Hq, Hkv, d, mp, r,
                                                  block))


def cluster_keys(k_cache, cache_len, is_retrieval, p_k, centroids,
                 iters: int = 1, n_recent: int = 2, r: int = 16,
                 block: int = 64, ws=None, tables=None):
    """k-means of the projected keys, seeded by `centroids` (updated in
    place). Returns the tables (cl_m [B], cl_off [B,n_ret,Lmax/block+1],
    cl_members [B,n_ret,Lmax]); `tables` may hold them already allocated."""
    lib = load()
    B, Hkv, Lmax, d = k_cache.shape
    Hq = len(is_retrieval)
    _dev(k_cache, torch.bfloat16, "k_cache")
    _dev(cache_len, torch.int32, "cache_len", (B,))
    m, mp = _mask(is_retrieval, Hq)
    n_ret = int(m.astype(bool).sum())
    _proj(p_k, n_ret, r, d, "p_k")
    _dev(centroids, torch.float32, "centroids", (B, n_ret, Lmax // block, r))
    dev = k_cache.device
    if tables is None:
        tables = (torch.zeros(B, dtype=torch.int32, device=dev),
                  torch.zeros((B, n_ret, Lmax // block + 1), dtype=torch.int32,
                              device=dev),
                  torch.zeros((B, n_ret, Lmax), dtype=torch.int32, device=dev))
    cl_m, cl_off, cl_mem = tables
    _dev(cl_m, torch.int32, "cl_m", (B,))
    _dev(cl_off, torch.int32, "cl_off", (B, n_ret, Lmax // block + 1))
    _dev(cl_mem, torch.int32, "cl_members", (B, n_ret, Lmax))
    nb = lib.rtp_cluster_workspace_bytes(B, Lmax, Hq, Hkv, d, mp, r, block)
    w = _workspace(nb, dev, ws)
    _check(lib.rtp_cluster_keys(
        _ptr(k_cache), _ptr(cache_len), B, Lmax, Hq, Hkv, d, mp, _ptr(p_k), r,
        block, n_recent, int(iters), _ptr(centroids), _ptr(cl_m),
        _ptr(cl_off), _ptr(cl_mem), _ptr(w), w.numel(), _stream(dev)),
        "rtp_cluster_keys")
    return tables


def decode_clustered_workspace_bytes(B: int, Lmax: int, Hq: int, Hkv: int,
                                     is_retrieval, top_k: int,
                                     n_recent: int = 2, r: int = 16,
                                     d: int = 128, block: int = 64) -> int:
    _, mp = _mask(is_retrieval, Hq)
    return int(load().rtp_decode_clustered_workspace_bytes(
        B, Lmax, Hq, Hkv, d, mp, r, block, top_k, n_recent))


def hybrid_attn_decode_clustered(q, k_cache, v_cache, cache_len, is_retrieval,
                                 window: int, p_q, centroids, tables,
                                 top_k: int, n_recent: int = 2, r: int = 16,
                                 block: int = 64, scale: float = 0.0,
                                 want_lse: bool = False,
                                 want_sel: bool = False, ws=None, out=None):
    """One decode step choosing among the clusters of cluster_keys.
    Returns out, or (out, lse, sel) when asked."""
    lib = load()
    B, Hq, d = q.shape
    _, Hkv, Lmax, _ = k_cache.shape
    _dev(q, torch.bfloat16, "q", (B, Hq, d))
    _dev(k_cache, torch.bfloat16, "k_cache", (B, Hkv, Lmax, d))
    _dev(v_cache, torch.bfloat16, "v_cache", (B, Hkv, Lmax, d))
    _dev(cache_len, torch.int32, "cache_len", (B,))
    m, mp = _mask(is_retrieval, Hq)
    n_ret = int(m.astype(bool).sum())
    cl_m, cl_off, cl_mem = tables
    if n_ret:
        _proj(p_q, n_ret, r, d, "p_q")
        _dev(centroids, torch.float32, "centroids",
             (B, n_ret, Lmax // block, r))
        _dev(cl_m, torch.int32, "cl_m", (B,))
        _dev(cl_off, torch.int32, "cl_off", (B, n_ret, Lmax // block + 1))
        _dev(cl_mem, torch.int32, "cl_members", (B, n_ret, Lmax))
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) \
        if want_lse else None
    so = torch.full((B, n_ret, top_k + 1 + n_recent), -1, dtype=torch.int32,
                    device=dev) if want_sel else None
    nb = lib.rtp_decode_clustered_workspace_bytes(B, Lmax, Hq, Hkv, d, mp, r,
                                                  block, top_k, n_recent)
    w = _workspace(nb, dev, ws)
    _check(lib.rtp_hybrid_attn_decode_clustered(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_len), B, Lmax, Hq,
        Hkv, d, mp, int(window), _ptr(p_q), _ptr(centroids), _ptr(cl_m),
        _ptr(cl_off), _ptr(cl_mem), r, block, top_k, n_recent, float(scale),
        _ptr(out), _ptr(lse), _ptr(so), _ptr(w), w.numel(), _stream(dev)),
        "rtp_hybrid_attn_decode_clustered")
    if want_lse or want_sel:
        return out, lse, so
    return out


class PagedCache:
    """A paged decode cache: k_pages / v_pages [n_pages, Hkv, 64, d] bf16 and
    a block table [B, max_blocks] int32 of page ids (device tensors)."""

    def __init__(self, k_pages, v_pages, block_table):
        n_pages, Hkv, blk, d = k_pages.shape
        _dev(k_pages, torch.bfloat16, "k_pages")
        _dev(v_pages, torch.bfloat16, "v_pages", (n_pages, Hkv, blk, d))
        _dev(block_table, torch.int32, "block_table")
        if blk != 64 or block_table.dim() != 2:
            raise ValueError("pages hold 64 tokens; block_table is [B, max_blocks]")
        self.k, self.v, self.table = k_pages, v_pages, block_table
        self.n_pages, self.Hkv, self.d = n_pages, Hkv, d
        self.B, self.max_blocks = block_table.shape
        self.Lmax = 64 * self.max_blocks


def build_centroids_paged(pc: PagedCache, cache_len, is_retrieval, p_k,
                          r: int = 16, block: int = 64, out=None):
    """build_centroids over a paged cache: [B, n_ret, max_blocks, r]."""
    lib = load()
    Hq = len(is_retrieval)
    _dev(cache_len, torch.int32, "cache_len", (pc.B,))
    m, mp = _mask(is_retrieval, Hq)
    n_ret = int(m.astype(bool).sum())
    _proj(p_k, n_ret, r, pc.d, "p_k")
    if out is None:
        out = torch.zeros((pc.B, n_ret, pc.max_blocks, r), dtype=torch.float32,
                          device=pc.k.device)
    _check(lib.rtp_build_centroids_paged(
        _ptr(pc.k), _ptr(pc.table), pc.max_blocks, pc.n_pages, _ptr(cache_len),
        pc.B, Hq, pc.Hkv, pc.d, mp, _ptr(p_k), r, block, _ptr(out),
        _stream(pc.k.device)), "rtp_build_centroids_paged")
    return out


def decode_append_paged(pc: PagedCache, cache_len, k_new, v_new,
                        is_retrieval, p_k=None, centroids=None, r: int = 16,
                        block: int = 64):
    lib = load()
    Hq = len(is_retrieval)
    _dev(cache_len, torch.int32, "cache_len", (pc.B,))
    _dev(k_new, torch.bfloat16, "k_new", (pc.B, pc.Hkv, pc.d))
    _dev(v_new, torch.bfloat16, "v_new", (pc.B, pc.Hkv, pc.d))
    m, mp = _mask(is_retrieval, Hq)
    n_ret = int(m.astype(bool).sum())
    if n_ret:
        _proj(p_k, n_ret, r, pc.d, "p_k")
        _dev(centroids, torch.float32, "centroids",
             (pc.B, n_ret, pc.max_blocks, r))
    _check(lib.rtp_decode_append_paged(
        _ptr(pc.k), _ptr(pc.v), _ptr(pc.table), pc.max_blocks, pc.n_pages,
        _ptr(cache_len), _ptr(k_new), _ptr(v_new), pc.B, Hq, pc.Hkv, pc.d, mp,
        _ptr(p_k) if n_ret else None, r, block,
        _ptr(centroids) if n_ret else None, _stream(pc.k.device)),
        "rtp_decode_append_paged")


def _decode_outputs(q, n_ret, top_k, n_recent, want_lse, want_sel, out):
    B, Hq, d = q.shape
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) \
        if want_lse else None
    so = torch.full((B, n_ret, top_k + 1 + n_recent), -1, dtype=torch.int32,
                    device=dev) if want_sel else None
    return out, lse, so


def hybrid_attn_decode_paged(q, pc: PagedCache, cache_len, is_retrieval,
                             window: int, p_q, centroids, top_k: int,
                             n_recent: int = 2, r: int = 16, block: int = 64,
                             scale: float = 0.0, want_lse: bool = False,
                             want_sel: bool = False, ws=None, out=None):
    lib = load()
    B, Hq, d = q.shape
    _dev(q, torch.bfloat16, "q", (pc.B, Hq, pc.d))
    _dev(cache_len, torch.int32, "cache_len", (pc.B,))
    m, mp = _mask(is_retrieval, Hq)
    n_ret = int(m.astype(bool).sum())
    if n_ret:
        _proj(p_q, n_ret, r, d, "p_q")
        _dev(centroids, torch.float32, "centroids",
             (B, n_ret, pc.max_blocks, r))
    out, lse, so = _decode_outputs(q, n_ret, top_k, n_recent, want_lse,
                                   want_sel, out)
    nb = lib.rtp_decode_workspace_bytes(B, pc.Lmax, Hq, pc.Hkv, d, mp, r,
                                        block, top_k, n_recent)
    w = _workspace(nb, q.device, ws)
    _check(lib.rtp_hybrid_attn_decode_paged(
        _ptr(q), _ptr(pc.k), _ptr(pc.v), _ptr(pc.table), pc.max_blocks,
        pc.n_pages, _ptr(cache_len), B, Hq, pc.Hkv, d, mp, int(window),
        _ptr(p_q), _ptr(centroids), r, block, top_k, n_recent, float(scale),
        _ptr(out), _ptr(lse), _ptr(so), _ptr(w), w.numel(),
        _stream(q.device)), "rtp_hybrid_attn_decode_paged")
    if want_lse or want_sel:
        return out, lse, so
    return out


def cluster_keys_paged(pc: PagedCache, cache_len, is_retrieval, p_k,
                       centroids, iters: int = 1, n_recent: int = 2,
                       r: int = 16, block: int = 64, ws=None, tables=None):
    lib = load()
    Hq = len(is_retrieval)
    _dev(cache_len, torch.int32, "cache_len", (pc.B,))
    m, mp = _mask(is_retrieval, Hq)
    n_ret = int(m.astype(bool).sum())
    _proj(p_k, n_ret, r, pc.d, "p_k")
    _dev(centroids, torch.float32, "centroids",
         (pc.B, n_ret, pc.max_blocks, r))
    dev = pc.k.device
    if tables is None:
        tables = (torch.zeros(pc.B, dtype=torch.int32, device=dev),
                  torch.zeros((pc.B, n_ret, pc.max_blocks + 1),
                              dtype=torch.int32, device=dev),
                  torch.zeros((pc.B, n_ret, pc.Lmax), dtype=torch.int32,
                              device=dev))
    cl_m, cl_off, cl_mem = tables
    nb = lib.rtp_cluster_workspace_bytes(pc.B, pc.Lmax, Hq, pc.Hkv, pc.d, mp,
                                         r, block)
    w = _workspace(nb, dev, ws)
    _check(lib.rtp_cluster_keys_paged(
        _ptr(pc.k), _ptr(pc.table), pc.max_blocks, pc.n_pages,
        _ptr(cache_len), pc.B, Hq, pc.Hkv, pc.d, mp, _ptr(p_k), r, block,
        n_recent, int(iters), _ptr(centroids), _ptr(cl_m), _ptr(cl_off),
        _ptr(cl_mem), _ptr(w), w.numel(), _stream(dev)),
        "rtp_cluster_keys_paged")
    return tables


def hybrid_attn_decode_clustered_paged(q, pc: PagedCache, cache_len,
                                       is_retrieval, window: int, p_q,
                                       centroids, tables, top_k: int,
                                       n_recent: int = 2, r: int = 16,
                                       block: int = 64, scale: float = 0.0,
                                       want_lse: bool = False,
                                       want_sel: bool = False, ws=None,
                                       out=None):
    lib = load()
    B, Hq, d = q.shape
    _dev(q, torch.bfloat16, "q", (pc.B, Hq, pc.d))
    _dev(cache_len, torch.int32, "cache_len", (pc.B,))
    m, mp = _mask(is_retrieval, Hq)
    n_ret = int(m.astype(bool).sum())
    cl_m, cl_off, cl_mem = tables
    if n_ret:
        _proj(p_q, n_ret, r, d, "p_q")
        _dev(centroids, torch.float32, "centroids",
             (B, n_ret, pc.max_blocks, r))
    out, lse, so = _decode_outputs(q, n_ret, top_k, n_recent, want_lse,
                                   want_sel, out)
    nb = lib.rtp_decode_clustered_workspace_bytes(B, pc.Lmax, Hq, pc.Hkv, d,
                                                  mp, r, block, top_k,
                                                  n_recent)
    w = _workspace(nb, q.device, ws)
    _check(lib.rtp_hybrid_attn_decode_clustered_paged(
        _ptr(q), _ptr(pc.k), _ptr(pc.v), _ptr(pc.table), pc.max_blocks,
        pc.n_pages, _ptr(cache_len), B, Hq, pc.Hkv, d, mp, int(window),
        _ptr(p_q), _ptr(centroids), _ptr(cl_m), _ptr(cl_off), _ptr(cl_mem),
        r, block, top_k, n_recent, float(scale), _ptr(out), _ptr(lse),
        _ptr(so), _ptr(w), w.numel(), _stream(q.device)),
        "rtp_hybrid_attn_decode_clustered_paged")
    if want_lse or want_sel:
        return out, lse, so
    return out
