"""PIVOT query-group indexer for MI355X (gfx950).

A thin ctypes binding over libpivot.so, whose C ABI is include/pivot.h.  This
module only marshals arguments: PyTorch provides device memory and the current
stream; every step of the indexer runs in the library's HIP kernels.  There is
no CPU fallback: importing works without the library, but every call raises if
libpivot.so has not been built (python -m top_token_selection_pivot_amd.build).

Method (arXiv:2607.24593, "PIVOT: Efficient Query-Group Indexing for
Token-Level Sparse Attention", English abstract): average each group of g
nearby queries into a proxy query, scan the full causal prefix once per group,
keep the proxy's top-C candidates, then either hand the proxy's top-k to every
member (Reuse) or let each member re-score the candidates and keep its own
top-k (Refine).
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

__all__ = [
    "DENSE", "REUSE", "REFINE", "PivotError", "library_path", "load",
    "indexer", "indexer_decode", "indexer_decode_paged", "indexer_varlen",
    "sparse_attention", "proxy_mean", "candidates", "decode_candidates",
    "workspace_size",
    "decode_workspace_size", "selftest_mfma_layout",
]

DENSE, REUSE, REFINE = 0, 1, 2
BF16, FP8 = 0, 1
_MODES = {"dense": DENSE, "reuse": REUSE, "refine": REFINE}

_HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; PIVOT_LIBRARY may name another build of the same ABI
_LIB_PATH = os.environ.get("PIVOT_LIBRARY") or os.path.join(_HERE, "libpivot.so")
_lib = None


class PivotError(RuntimeError):
    pass


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libpivot.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise PivotError(f"{_LIB_PATH} is missing: build it with "
                         "`python -m top_token_selection_pivot_amd.build`")
    L = C.CDLL(_LIB_PATH)
    vp, fp, ip, sz, i = C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_int
    L.pivot_version.restype = i
    L.pivot_status_string.restype = C.c_char_p
    L.pivot_status_string.argtypes = [i]
    L.pivot_last_error.restype = C.c_char_p
    L.pivot_workspace_size.restype = sz
    L.pivot_workspace_size.argtypes = [i] * 8
    L.pivot_workspace_min_size.restype = sz
    L.pivot_workspace_min_size.argtypes = [i] * 8
    L.pivot_indexer.restype = i
    L.pivot_indexer.argtypes = [vp, fp, fp, vp, fp] + [i] * 8 + [ip, vp, sz, vp]
    L.pivot_candidates.restype = i
    L.pivot_candidates.argtypes = [vp, fp, fp, vp, fp] + [i] * 8 + [ip, vp, sz, vp]
    L.pivot_proxy_mean.restype = i
    L.pivot_proxy_mean.argtypes = [vp, fp, fp] + [i] * 5 + [vp, fp, fp, vp]
    L.pivot_decode_workspace_size.restype = sz
    L.pivot_decode_workspace_size.argtypes = [i] * 9
    L.pivot_indexer_decode.restype = i
    L.pivot_indexer_decode.argtypes = [vp, fp, fp, vp, fp, ip] + [i] * 9 + [ip, vp, sz, vp]
    L.pivot_indexer_window.restype = i
    L.pivot_indexer_window.argtypes = [vp, fp, fp, vp, fp] + [i] * 10 + [ip, vp, sz, vp]
    L.pivot_indexer_decode_window.restype = i
    L.pivot_indexer_decode_window.argtypes = [vp, fp, fp, vp, fp, ip] + [i] * 11 + [ip, vp, sz, vp]
    L.pivot_sparse_attention_workspace_size.restype = sz
    L.pivot_sparse_attention_workspace_size.argtypes = [i] * 4
    L.pivot_sparse_attention.restype = i
    L.pivot_sparse_attention.argtypes = [vp, vp, vp, ip] + [i] * 6 + [C.c_longlong, i, C.c_float,
                                                                      fp, vp, sz, vp]
    L.pivot_varlen_workspace_size.restype = sz
    L.pivot_varlen_workspace_size.argtypes = [vp] + [i] * 8
    L.pivot_indexer_varlen.restype = i
    L.pivot_indexer_varlen.argtypes = [vp, fp, fp, vp, fp, vp] + [i] * 10 + [ip, vp, sz, vp]
    L.pivot_decode_candidates.restype = i
    L.pivot_indexer_decode_paged.argtypes = [vp, fp, fp, vp, fp, i, i, ip, i, ip] + [i] * 10 + [ip, vp, sz, vp]
    L.pivot_indexer_decode_paged.restype = i
    L.pivot_decode_candidates.argtypes = [vp, fp, fp, vp, fp, ip] + [i] * 9 + [ip, vp, sz, vp]
    L.pivot_profile_enable.restype = i
    L.pivot_profile_enable.argtypes = [i]
    L.pivot_profile_read.restype = i
    L.pivot_profile_read.argtypes = [vp, vp, i]
    L.pivot_selftest_mfma_layout.restype = i
    L.pivot_selftest_mfma_layout.argtypes = [ip, vp]
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        L = load()
        raise PivotError(f"{L.pivot_status_string(status).decode()}: "
                         f"{L.pivot_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _mode(mode) -> int:
    return _MODES[mode] if isinstance(mode, str) else int(mode)


def _dtype_of(q: torch.Tensor) -> int:
    if q.element_size() == 2:
        return BF16
    if q.element_size() == 1:
        return FP8
    raise PivotError(f"unsupported code type {q.dtype}: use bf16 (2-byte) or fp8 e4m3 (1-byte)")


def _dev(t: Optional[torch.Tensor], name: str, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise PivotError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise PivotError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise PivotError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def workspace_size(L, H, D, g, topk, C, mode, dtype) -> int:
    return load().pivot_workspace_size(L, H, D, g, topk, C, _mode(mode), dtype)


def decode_workspace_size(B, Lmax, H, D, g, topk, C, mode, dtype) -> int:
    return load().pivot_decode_workspace_size(B, Lmax, H, D, g, topk, C, _mode(mode), dtype)


def _workspace(nbytes: int, device, workspace, min_bytes: Optional[int] = None):
    """The caller's workspace (at least min_bytes, default nbytes) or a new one of nbytes."""
    if workspace is not None:
        need = nbytes if min_bytes is None else min_bytes
        if workspace.numel() * workspace.element_size() < need:
            raise PivotError(f"workspace of {workspace.numel() * workspace.element_size()} bytes "
                             f"is below the minimum {need}")
        return workspace
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


WINDOW_MODES = {"shared": 0, "excluded": 1}


def _window_mode(wm) -> int:
    return WINDOW_MODES[wm] if isinstance(wm, str) else int(wm)


def indexer(q, w, k, *, g: int, topk: int, C: int = 0, mode="refine", q_scale=None,
            k_scale=None, out=None, workspace=None, stream=None, window: int = 0,
            window_mode="shared") -> torch.Tensor:
    """Prefill indexer for one sequence.

    q [L,H,D] bf16 or fp8 codes, w [L,H] float32, k [L,D] codes; fp8 needs
    q_scale [L] and k_scale [L] float32.  Returns int32 [L, topk]: ascending
    selected positions, -1 padded.  window > 0 adds the sliding window of that
    size to every row (window_mode "shared" or "excluded", as in
    pivot_indexer_window) and returns [L, topk + window].
    """
    L = load()
    q, w, k = _dev(q, "q"), _dev(w, "w", torch.float32), _dev(k, "k")
    q_scale, k_scale = _dev(q_scale, "q_scale", torch.float32), _dev(k_scale, "k_scale", torch.float32)
    Lq, H, D = q.shape
    dt = _dtype_of(q)
    m = _mode(mode)
    if out is None:
        out = torch.empty((Lq, topk + window), dtype=torch.int32, device=q.device)
    ws = _workspace(L.pivot_workspace_size(Lq, H, D, g, topk, C, m, dt), q.device, workspace,
                    L.pivot_workspace_min_size(Lq, H, D, g, topk, C, m, dt))
    nbytes = ws.numel() * ws.element_size()
    if window:
        _check(L.pivot_indexer_window(_ptr(q), _ptr(q_scale), _ptr(w), _ptr(k), _ptr(k_scale), Lq,
                                      H, D, g, topk, C, m, dt, window, _window_mode(window_mode),
                                      _ptr(out), _ptr(ws), nbytes, _stream(stream)))
    else:
        _check(L.pivot_indexer(_ptr(q), _ptr(q_scale), _ptr(w), _ptr(k), _ptr(k_scale), Lq, H, D,
                               g, topk, C, m, dt, _ptr(out), _ptr(ws), nbytes, _stream(stream)))
    return out


def indexer_varlen(q, w, k, cu_seqlens, *, g: int, topk: int, C: int = 0, mode="refine",
                   q_scale=None, k_scale=None, window: int = 0, window_mode="shared", out=None,
                   workspace=None, stream=None) -> torch.Tensor:
    """Several prefill sequences in one call (pivot_indexer_varlen): q [T,H,D],
    w [T,H], k [T,D] hold the sequences back to back; cu_seqlens (host ints,
    nseq + 1 offsets starting at 0) delimits them.  Returns int32
    [T, topk + window]; each sequence's rows are those of indexer() on it alone."""
    import numpy as np
    L = load()
    q, w, k = _dev(q, "q"), _dev(w, "w", torch.float32), _dev(k, "k")
    q_scale, k_scale = _dev(q_scale, "q_scale", torch.float32), _dev(k_scale, "k_scale", torch.float32)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    nseq = cu.shape[0] - 1
    T, H, D = q.shape
    dt = _dtype_of(q)
    m = _mode(mode)
    if out is None:
        out = torch.empty((T, topk + window), dtype=torch.int32, device=q.device)
    ws = _workspace(L.pivot_varlen_workspace_size(cu.ctypes.data, nseq, H, D, g, topk, C, m, dt),
                    q.device, workspace)
    _check(L.pivot_indexer_varlen(_ptr(q), _ptr(q_scale), _ptr(w), _ptr(k), _ptr(k_scale),
                                  cu.ctypes.data, nseq, H, D, g, topk, C, m, dt, window,
                                  _window_mode(window_mode), _ptr(out), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream)))
    return out


def candidates(q, w, k, *, g: int, topk: int, C: int = 0, mode="refine", q_scale=None,
               k_scale=None, workspace=None, stream=None) -> torch.Tensor:
    """Every group's proxy top-m (m = C for Refine, topk for Reuse): int32 [G, m]."""
    L = load()
    q, w, k = _dev(q, "q"), _dev(w, "w", torch.float32), _dev(k, "k")
    Lq, H, D = q.shape
    dt = _dtype_of(q)
    m = _mode(mode)
    G = (Lq + g - 1) // g
    cand = torch.empty((G, C if m == REFINE else topk), dtype=torch.int32, device=q.device)
    ws = _workspace(L.pivot_workspace_size(Lq, H, D, g, topk, C, m, dt), q.device, workspace,
                    L.pivot_workspace_min_size(Lq, H, D, g, topk, C, m, dt))
    _check(L.pivot_candidates(_ptr(q), _ptr(q_scale), _ptr(w), _ptr(k), _ptr(k_scale), Lq, H, D,
                              g, topk, C, m, dt, _ptr(cand), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(stream)))
    return cand


def proxy_mean(q, w, g: int, q_scale=None, stream=None):
    """Proxy codes [G,H,D] (same code type as q), proxy scales [G] and weights [G,H]."""
    L = load()
    q, w = _dev(q, "q"), _dev(w, "w", torch.float32)
    Lq, H, D = q.shape
    dt = _dtype_of(q)
    G = (Lq + g - 1) // g
    qbar = torch.empty((G, H, D), dtype=q.dtype, device=q.device)
    qs = torch.empty(G, dtype=torch.float32, device=q.device)
    wbar = torch.empty((G, H), dtype=torch.float32, device=q.device)
    _check(L.pivot_proxy_mean(_ptr(q), _ptr(q_scale), _ptr(w), Lq, H, D, g, dt, _ptr(qbar),
                              _ptr(qs), _ptr(wbar), _stream(stream)))
    return qbar, qs, wbar


def indexer_decode(q, w, k_cache, cache_len, *, topk: int, C: int = 0, mode="refine",
                   q_scale=None, k_scale=None, out=None, workspace=None,
                   stream=None, window: int = 0, window_mode="shared") -> torch.Tensor:
    """One MTP decode step: q [B,g,H,D], w [B,g,H], k_cache [B,Lmax,D],
    cache_len [B] int32 (device); fp8 needs q_scale [B,g], k_scale [B,Lmax].
    Returns int32 [B, g, topk] ([B, g, topk + window] with a window)."""
    L = load()
    q, w, k_cache = _dev(q, "q"), _dev(w, "w", torch.float32), _dev(k_cache, "k_cache")
    cache_len = _dev(cache_len, "cache_len", torch.int32)
    B, g, H, D = q.shape
    Lmax = k_cache.shape[1]
    dt = _dtype_of(q)
    m = _mode(mode)
    if out is None:
        out = torch.empty((B, g, topk + window), dtype=torch.int32, device=q.device)
    ws = _workspace(L.pivot_decode_workspace_size(B, Lmax, H, D, g, topk, C, m, dt), q.device,
                    workspace)
    nbytes = ws.numel() * ws.element_size()
    if window:
        _check(L.pivot_indexer_decode_window(
            _ptr(q), _ptr(q_scale), _ptr(w), _ptr(k_cache), _ptr(k_scale), _ptr(cache_len), B,
            Lmax, H, D, g, topk, C, m, dt, window, _window_mode(window_mode), _ptr(out), _ptr(ws),
            nbytes, _stream(stream)))
    else:
        _check(L.pivot_indexer_decode(_ptr(q), _ptr(q_scale), _ptr(w), _ptr(k_cache),
                                      _ptr(k_scale), _ptr(cache_len), B, Lmax, H, D, g, topk, C, m,
                                      dt, _ptr(out), _ptr(ws), nbytes, _stream(stream)))
    return out


def indexer_decode_paged(q, w, k_pages, block_table, cache_len, *, topk: int, C: int = 0,
                         mode="refine", q_scale=None, k_scale=None, window: int = 0,
                         window_mode="shared", out=None, workspace=None,
                         stream=None) -> torch.Tensor:
    """One MTP decode step over a paged key cache (pivot_indexer_decode_paged).

    k_pages [num_pages, page_size, D] codes (fp8: k_scale [num_pages,
    page_size]); block_table [B, max_pages] int32 page ids (device); position
    p of sequence b is row p % page_size of page block_table[b, p //
    page_size].  Other arguments as for indexer_decode.  Returns int32
    [B, g, topk + window]."""
    L = load()
    q, w, k_pages = _dev(q, "q"), _dev(w, "w", torch.float32), _dev(k_pages, "k_pages")
    block_table = _dev(block_table, "block_table", torch.int32)
    cache_len = _dev(cache_len, "cache_len", torch.int32)
    B, g, H, D = q.shape
    num_pages, page_size = k_pages.shape[0], k_pages.shape[1]
    max_pages = block_table.shape[1]
    dt = _dtype_of(q)
    m = _mode(mode)
    if out is None:
        out = torch.empty((B, g, topk + window), dtype=torch.int32, device=q.device)
    ws = _workspace(L.pivot_decode_workspace_size(B, max_pages * page_size, H, D, g, topk, C, m, dt),
                    q.device, workspace)
    _check(L.pivot_indexer_decode_paged(
        _ptr(q), _ptr(q_scale), _ptr(w), _ptr(k_pages), _ptr(k_scale), num_pages, page_size,
        _ptr(block_table), max_pages, _ptr(cache_len), B, H, D, g, topk, C, m, dt, window,
        _window_mode(window_mode), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))
    return out


def decode_candidates(q, w, k_cache, cache_len, *, topk: int, C: int = 0, mode="refine",
                      q_scale=None, k_scale=None, workspace=None, stream=None) -> torch.Tensor:
    """Every sequence's proxy top-m for one decode step: int32 [B, m]."""
    L = load()
    q, w, k_cache = _dev(q, "q"), _dev(w, "w", torch.float32), _dev(k_cache, "k_cache")
    cache_len = _dev(cache_len, "cache_len", torch.int32)
    B, g, H, D = q.shape
    Lmax = k_cache.shape[1]
    dt = _dtype_of(q)
    m = _mode(mode)
    cand = torch.empty((B, C if m == REFINE else topk), dtype=torch.int32, device=q.device)
    ws = _workspace(L.pivot_decode_workspace_size(B, Lmax, H, D, g, topk, C, m, dt), q.device,
                    workspace)
    _check(L.pivot_decode_candidates(_ptr(q), _ptr(q_scale), _ptr(w), _ptr(k_cache),
                                     _ptr(k_scale), _ptr(cache_len), B, Lmax, H, D, g, topk, C,
                                     m, dt, _ptr(cand), _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream(stream)))
    return cand


def sparse_attention(q, k, v, idx, *, rows_per_seq: Optional[int] = None, seq_len=None,
                     scale=None, out=None, workspace=None, stream=None) -> torch.Tensor:
    """Sparse main attention over the selected positions (pivot_sparse_attention).

    q [R,Hq,d] bf16; k [N,d] and v [N,dv] bf16 (one sequence) or [B,S,d] and
    [B,S,dv] (row r reads sequence r // rows_per_seq); idx [R,nidx] int32
    positions (-1 and out-of-range entries are skipped).  Returns float32
    [R,Hq,dv]."""
    import math
    L = load()
    q, k, v = _dev(q, "q"), _dev(k, "k"), _dev(v, "v")
    idx = _dev(idx, "idx", torch.int32)
    R, Hq, d = q.shape
    dv = v.shape[-1]
    if k.dim() == 2:
        stride, nkeys = 0, k.shape[0]
        rows_per_seq = R if rows_per_seq is None else rows_per_seq
    else:
        stride, nkeys = k.shape[1], k.shape[1]
        if rows_per_seq is None:
            raise ValueError("rows_per_seq is needed with per-sequence k/v")
    seq_len = nkeys if seq_len is None else seq_len
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    nidx = idx.shape[1]
    if out is None:
        out = torch.empty((R, Hq, dv), dtype=torch.float32, device=q.device)
    need = L.pivot_sparse_attention_workspace_size(R, Hq, dv, nidx)
    ws = _workspace(need, q.device, workspace) if need else None
    _check(L.pivot_sparse_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(idx), R, Hq, d, dv, nidx,
                                    rows_per_seq, stride, seq_len, float(scale), _ptr(out),
                                    _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                    _stream(stream)))
    return out


def selftest_mfma_layout(device="cuda") -> torch.Tensor:
    """[3, 2, 64, 16] int32: row / column / pairing probes for bf16 and fp8 tiles."""
    L = load()
    out = torch.zeros((3, 2, 64, 16), dtype=torch.int32, device=device)
    _check(L.pivot_selftest_mfma_layout(_ptr(out), _stream(None)))
    return out


KERNEL_CLASSES = ("proxy_mean", "scan", "select", "refine_score", "member_select", "broadcast",
                  "decode_scan", "window", "attention")


def profile_enable(on: bool = True) -> None:
    """Bracket every library launch with HIP events on its stream (see profile_read)."""
    _check(load().pivot_profile_enable(1 if on else 0))


def profile_read() -> dict:
    """{kernel class: (milliseconds, launches)} since the last read; clears the record."""
    import numpy as np
    n = len(KERNEL_CLASSES)
    ms = np.zeros(n, np.float64)
    cnt = np.zeros(n, np.int64)
    _check(load().pivot_profile_read(ms.ctypes.data, cnt.ctypes.data, n))
    return {k: (float(ms[i]), int(cnt[i])) for i, k in enumerate(KERNEL_CLASSES)}
