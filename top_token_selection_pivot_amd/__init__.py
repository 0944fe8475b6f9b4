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
    "indexer", "indexer_decode", "indexer_decode_paged", "indexer_varlen", "score_rows",
    "indexer_layers", "indexer_decode_layers", "indexer_decode_noalloc",
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
    L.pivot_last_error_detail.restype = C.c_char_p
    L.pivot_workspace_size.restype = sz
    L.pivot_workspace_size.argtypes = [i] * 8
    L.pivot_workspace_min_size.restype = sz
    L.pivot_workspace_min_size.argtypes = [i] * 8
    L.pivot_indexer.restype = i
    L.pivot_indexer.argtypes = [vp, fp, fp, vp, fp] + [i] * 8 + [ip, fp, vp, sz, vp]
    L.pivot_candidates.restype = i
    L.pivot_candidates.argtypes = [vp, fp, fp, vp, fp] + [i] * 8 + [ip, vp, sz, vp]
    L.pivot_proxy_mean.restype = i
    L.pivot_proxy_mean.argtypes = [vp, fp, fp] + [i] * 5 + [vp, fp, fp, vp]
    L.pivot_decode_workspace_size.restype = sz
    L.pivot_decode_workspace_size.argtypes = [i] * 9
    L.pivot_indexer_decode.restype = i
    L.pivot_indexer_decode.argtypes = [vp, fp, fp, vp, fp, ip] + [i] * 9 + [ip, fp, vp, sz, vp]
    L.pivot_indexer_decode_noalloc.restype = i
    L.pivot_indexer_decode_noalloc.argtypes = [vp, fp, fp, vp, fp, ip] + [i] * 9 + [ip, fp, vp]
    L.pivot_noalloc_scratch_bytes.restype = sz
    L.pivot_noalloc_scratch_bytes.argtypes = []
    L.pivot_indexer_layers.restype = i
    L.pivot_indexer_layers.argtypes = [i, vp, vp, vp, vp, vp, vp] + [i] * 8 + [vp, vp, sz, vp]
    L.pivot_indexer_decode_layers.restype = i
    L.pivot_indexer_decode_layers.argtypes = [i, vp, vp, vp, vp, vp, vp, ip] + [i] * 9 + [vp, vp, sz, vp]
    L.pivot_dbg_score_rows.restype = i
    L.pivot_dbg_score_rows.argtypes = [vp, fp, fp, vp, fp] + [i] * 9 + [fp, C.c_longlong, vp]
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
                         f"{L.pivot_last_error_detail().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _mode(mode) -> int:
    m = _MODES.get(mode, -1) if isinstance(mode, str) else int(mode)
    if m not in (DENSE, REUSE, REFINE):
        raise PivotError(f"mode {mode!r} is not dense, reuse or refine")
    return m


_CODE_TYPES = {torch.bfloat16: BF16, torch.float8_e4m3fn: FP8}


def _dtype_of(q: torch.Tensor) -> int:
    dt = _CODE_TYPES.get(q.dtype)
    if dt is None:
        raise PivotError(f"unsupported code type {q.dtype}: use torch.bfloat16 or torch.float8_e4m3fn")
    return dt


def _expect(t: Optional[torch.Tensor], name: str, shape, dtype=None, optional=False):
    """Shape and dtype checks that run before anything touches the device."""
    if t is None:
        if optional:
            return None
        raise PivotError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise PivotError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise PivotError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise PivotError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _scales(dt: int, q_scale, k_scale, qs_shape, ks_shape):
    if dt == FP8:
        _expect(q_scale, "q_scale", qs_shape, torch.float32)
        _expect(k_scale, "k_scale", ks_shape, torch.float32)
    elif q_scale is not None or k_scale is not None:
        raise PivotError("bf16 inputs take no q_scale / k_scale")


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


def _on_device(**tensors):
    for name, t in tensors.items():
        _dev(t, name)


def workspace_size(L, H, D, g, topk, C, mode, dtype) -> int:
    return load().pivot_workspace_size(L, H, D, g, topk, C, _mode(mode), dtype)


def decode_workspace_size(B, Lmax, H, D, g, topk, C, mode, dtype) -> int:
    return load().pivot_decode_workspace_size(B, Lmax, H, D, g, topk, C, _mode(mode), dtype)


def _workspace(nbytes: int, device, workspace, min_bytes: Optional[int] = None):
    """The caller's workspace (at least min_bytes, default nbytes) or a new one of nbytes."""
    if workspace is not None:
        if workspace.dtype != torch.uint8 or workspace.dim() != 1:
            raise PivotError("workspace must be a 1-D torch.uint8 tensor")
        _dev(workspace, "workspace")
        need = nbytes if min_bytes is None else min_bytes
        if workspace.numel() < need:
            raise PivotError(f"workspace of {workspace.numel()} bytes is below the minimum {need}")
        return workspace
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


WINDOW_MODES = {"shared": 0, "excluded": 1}


def _window_mode(wm) -> int:
    m = WINDOW_MODES.get(wm, -1) if isinstance(wm, str) else int(wm)
    if m not in (0, 1):
        raise PivotError(f"window_mode {wm!r} is not shared or excluded")
    return m


def _prefill_inputs(q, w, k, q_scale, k_scale):
    """Checks one sequence's q [L,H,D], w [L,H], k [L,D] (+ fp8 scales [L])."""
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise PivotError("q must be a [L, H, D] tensor")
    dt = _dtype_of(q)
    Lq, H, D = q.shape
    _expect(w, "w", (Lq, H), torch.float32)
    _expect(k, "k", (Lq, D), q.dtype)
    _scales(dt, q_scale, k_scale, (Lq,), (Lq,))
    return dt, Lq, H, D


def _out(out, name, shape, dtype, device):
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _expect(out, name, shape, dtype)
    _dev(out, name)
    return out


def indexer(q, w, k, *, g: int, topk: int, C: int = 0, mode="refine", q_scale=None,
            k_scale=None, out=None, workspace=None, stream=None, window: int = 0,
            window_mode="shared", out_scores=None, return_scores: bool = False):
    """Prefill indexer for one sequence.

    q [L,H,D] bf16 or fp8 (float8_e4m3fn) codes, w [L,H] float32, k [L,D]
    codes of q's type; fp8 needs q_scale [L] and k_scale [L] float32.  Returns
    int32 [L, topk]: ascending selected positions, -1 padded.  window > 0 adds
    the sliding window of that size to every row (window_mode "shared" or
    "excluded", as in pivot_indexer_window) and returns [L, topk + window].
    With return_scores (or a float32 [L, topk] out_scores; no window) the
    score of every selected position is written too and (out, scores) is
    returned.
    """
    L = load()
    dt, Lq, H, D = _prefill_inputs(q, w, k, q_scale, k_scale)
    m = _mode(mode)
    if window < 0:
        raise PivotError("window must be >= 0")
    wm = _window_mode(window_mode)
    out = _out(out, "out", (Lq, topk + window), torch.int32, q.device)
    want = return_scores or out_scores is not None
    if want:
        if window:
            raise PivotError("scores are returned without a window only")
        out_scores = _out(out_scores, "out_scores", (Lq, topk), torch.float32, q.device)
    _on_device(q=q, w=w, k=k, q_scale=q_scale, k_scale=k_scale)
    ws = _workspace(L.pivot_workspace_size(Lq, H, D, g, topk, C, m, dt), q.device, workspace,
                    L.pivot_workspace_min_size(Lq, H, D, g, topk, C, m, dt))
    nbytes = ws.numel()
    if window:
        _check(L.pivot_indexer_window(_ptr(q), _ptr(q_scale), _ptr(w), _ptr(k), _ptr(k_scale), Lq,
                                      H, D, g, topk, C, m, dt, window, wm,
                                      _ptr(out), _ptr(ws), nbytes, _stream(stream)))
    else:
        _check(L.pivot_indexer(_ptr(q), _ptr(q_scale), _ptr(w), _ptr(k), _ptr(k_scale), Lq, H, D,
                               g, topk, C, m, dt, _ptr(out), _ptr(out_scores), _ptr(ws), nbytes,
                               _stream(stream)))
    return (out, out_scores) if want else out


def _ptr_array(ts):
    import numpy as np
    return np.ascontiguousarray([0 if t is None else t.data_ptr() for t in ts], dtype=np.uint64)


def _full_flags(full, nl):
    import numpy as np
    f = np.ascontiguousarray(np.asarray(full, dtype=np.int32).reshape(-1))
    if f.shape[0] != nl:
        raise PivotError(f"full must hold one flag per layer ({nl}), got {f.shape[0]}")
    if nl < 1 or not f[0]:
        raise PivotError("layer 0 must run its indexer (full[0] true)")
    return f


def indexer_layers(qs, ws, ks, *, full, g: int, topk: int, C: int = 0, mode="refine", q_scales=None,
                   k_scales=None, outs=None, workspace=None, stream=None):
    """Cross-layer index reuse stacked on the prefill indexer
    (pivot_indexer_layers): per layer l the tensors qs[l] [L,H,D], ws[l]
    [L,H], ks[l] [L,D] (fp8: q_scales[l], k_scales[l] [L]); full[l] true runs
    the indexer, false reuses the rows of the nearest full layer before it
    (only outs[l] is touched for such a layer, and its inputs may be None).
    Returns the list of int32 [L, topk] rows per layer."""
    L = load()
    nl = len(qs)
    f = _full_flags(full, nl)
    if len(ws) != nl or len(ks) != nl:
        raise PivotError("qs, ws and ks need one entry per layer")
    q_scales = q_scales or [None] * nl
    k_scales = k_scales or [None] * nl
    shape = None
    for l in range(nl):
        if not f[l]:
            continue
        dt, Lq, H, D = _prefill_inputs(qs[l], ws[l], ks[l], q_scales[l], k_scales[l])
        if shape is not None and (dt, Lq, H, D) != shape:
            raise PivotError(f"layer {l}: every full layer needs the same code type and shape")
        shape = (dt, Lq, H, D)
        _on_device(q=qs[l], w=ws[l], k=ks[l], q_scale=q_scales[l], k_scale=k_scales[l])
    dt, Lq, H, D = shape
    m = _mode(mode)
    dev = qs[0].device
    outs = outs or [None] * nl
    outs = [_out(o, f"outs[{l}]", (Lq, topk), torch.int32, dev) for l, o in enumerate(outs)]
    wsp = _workspace(L.pivot_workspace_size(Lq, H, D, g, topk, C, m, dt), dev, workspace,
                     L.pivot_workspace_min_size(Lq, H, D, g, topk, C, m, dt))
    arrs = [_ptr_array(x) for x in (qs, q_scales, ws, ks, k_scales, outs)]
    fp8 = dt == FP8
    _check(L.pivot_indexer_layers(nl, f.ctypes.data, arrs[0].ctypes.data,
                                  arrs[1].ctypes.data if fp8 else None, arrs[2].ctypes.data,
                                  arrs[3].ctypes.data, arrs[4].ctypes.data if fp8 else None, Lq, H, D,
                                  g, topk, C, m, dt, arrs[5].ctypes.data, _ptr(wsp), wsp.numel(),
                                  _stream(stream)))
    return outs


def indexer_decode_layers(qs, ws, ks, cache_len, *, full, topk: int, C: int = 0, mode="refine",
                          q_scales=None, k_scales=None, outs=None, workspace=None, stream=None):
    """Cross-layer index reuse stacked on the decode step
    (pivot_indexer_decode_layers): per layer qs[l] [B,g,H,D], ws[l] [B,g,H],
    ks[l] [B,Lmax,D] (fp8: scales); cache_len [B] shared.  Returns the list
    of int32 [B, g, topk] rows per layer."""
    L = load()
    nl = len(qs)
    f = _full_flags(full, nl)
    q_scales = q_scales or [None] * nl
    k_scales = k_scales or [None] * nl
    shape = None
    for l in range(nl):
        if not f[l]:
            continue
        sh = _decode_inputs(qs[l], ws[l], ks[l], cache_len, q_scales[l], k_scales[l])
        if shape is not None and sh != shape:
            raise PivotError(f"layer {l}: every full layer needs the same code type and shape")
        shape = sh
        _on_device(q=qs[l], w=ws[l], k_cache=ks[l], cache_len=cache_len, q_scale=q_scales[l],
                   k_scale=k_scales[l])
    dt, B, g, H, D, Lmax = shape
    m = _mode(mode)
    dev = qs[0].device
    outs = outs or [None] * nl
    outs = [_out(o, f"outs[{l}]", (B, g, topk), torch.int32, dev) for l, o in enumerate(outs)]
    wsp = _workspace(L.pivot_decode_workspace_size(B, Lmax, H, D, g, topk, C, m, dt), dev, workspace)
    arrs = [_ptr_array(x) for x in (qs, q_scales, ws, ks, k_scales, outs)]
    fp8 = dt == FP8
    _check(L.pivot_indexer_decode_layers(nl, f.ctypes.data, arrs[0].ctypes.data,
                                         arrs[1].ctypes.data if fp8 else None, arrs[2].ctypes.data,
                                         arrs[3].ctypes.data, arrs[4].ctypes.data if fp8 else None,
                                         _ptr(cache_len), B, Lmax, H, D, g, topk, C, m, dt,
                                         arrs[5].ctypes.data, _ptr(wsp), wsp.numel(), _stream(stream)))
    return outs


def indexer_varlen(q, w, k, cu_seqlens, *, g: int, topk: int, C: int = 0, mode="refine",
                   q_scale=None, k_scale=None, window: int = 0, window_mode="shared", out=None,
                   workspace=None, stream=None) -> torch.Tensor:
    """Several prefill sequences in one call (pivot_indexer_varlen): q [T,H,D],
    w [T,H], k [T,D] hold the sequences back to back; cu_seqlens (host ints,
    nseq + 1 offsets starting at 0 and ending at T) delimits them.  Returns
    int32 [T, topk + window]; each sequence's rows are those of indexer() on it
    alone."""
    import numpy as np
    L = load()
    dt, T, H, D = _prefill_inputs(q, w, k, q_scale, k_scale)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    if cu.ndim != 1 or cu.shape[0] < 2 or cu[0] != 0 or cu[-1] != T:
        raise PivotError(f"cu_seqlens must be 1-D offsets from 0 to {T}")
    nseq = cu.shape[0] - 1
    m = _mode(mode)
    wm = _window_mode(window_mode)
    out = _out(out, "out", (T, topk + window), torch.int32, q.device)
    _on_device(q=q, w=w, k=k, q_scale=q_scale, k_scale=k_scale)
    lmax = int(np.max(np.diff(cu))) if nseq else 0
    ws = _workspace(L.pivot_varlen_workspace_size(cu.ctypes.data, nseq, H, D, g, topk, C, m, dt),
                    q.device, workspace,
                    L.pivot_workspace_min_size(lmax, H, D, g, topk, C, m, dt) if lmax else 256)
    _check(L.pivot_indexer_varlen(_ptr(q), _ptr(q_scale), _ptr(w), _ptr(k), _ptr(k_scale),
                                  cu.ctypes.data, nseq, H, D, g, topk, C, m, dt, window, wm,
                                  _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def candidates(q, w, k, *, g: int, topk: int, C: int = 0, mode="refine", q_scale=None,
               k_scale=None, workspace=None, stream=None) -> torch.Tensor:
    """Every group's proxy top-m (m = C for Refine, topk for Reuse): int32 [G, m]."""
    L = load()
    dt, Lq, H, D = _prefill_inputs(q, w, k, q_scale, k_scale)
    m = _mode(mode)
    G = (Lq + g - 1) // g
    _on_device(q=q, w=w, k=k, q_scale=q_scale, k_scale=k_scale)
    cand = torch.empty((G, C if m == REFINE else topk), dtype=torch.int32, device=q.device)
    ws = _workspace(L.pivot_workspace_size(Lq, H, D, g, topk, C, m, dt), q.device, workspace,
                    L.pivot_workspace_min_size(Lq, H, D, g, topk, C, m, dt))
    _check(L.pivot_candidates(_ptr(q), _ptr(q_scale), _ptr(w), _ptr(k), _ptr(k_scale), Lq, H, D,
                              g, topk, C, m, dt, _ptr(cand), _ptr(ws), ws.numel(), _stream(stream)))
    return cand


def proxy_mean(q, w, g: int, q_scale=None, stream=None):
    """Proxy codes [G,H,D] (same code type as q), proxy scales [G] and weights [G,H]."""
    L = load()
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise PivotError("q must be a [L, H, D] tensor")
    dt = _dtype_of(q)
    Lq, H, D = q.shape
    _expect(w, "w", (Lq, H), torch.float32)
    if dt == FP8:
        _expect(q_scale, "q_scale", (Lq,), torch.float32)
    elif q_scale is not None:
        raise PivotError("bf16 inputs take no q_scale")
    _on_device(q=q, w=w, q_scale=q_scale)
    G = (Lq + g - 1) // g
    qbar = torch.empty((G, H, D), dtype=q.dtype, device=q.device)
    qs = torch.empty(G, dtype=torch.float32, device=q.device)
    wbar = torch.empty((G, H), dtype=torch.float32, device=q.device)
    _check(L.pivot_proxy_mean(_ptr(q), _ptr(q_scale), _ptr(w), Lq, H, D, g, dt, _ptr(qbar),
                              _ptr(qs), _ptr(wbar), _stream(stream)))
    return qbar, qs, wbar


def score_rows(q, w, k, *, row_begin: int = 0, row_end: Optional[int] = None, pos_mul: int = 1,
               pos_add: int = 0, q_scale=None, k_scale=None, stream=None) -> torch.Tensor:
    """Indexer score rows as the full-prefix scan computes them
    (pivot_dbg_score_rows): q [R,H,D] query rows (raw queries, or the proxies
    of proxy_mean with pos_mul = g, pos_add = g - 1), w [R,H], k [Lk,D]; row r
    sees keys 0..min(r*pos_mul + pos_add, Lk-1).  Returns float32
    [row_end - row_begin, Lk]; entries past a row's last key are NaN."""
    L = load()
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise PivotError("q must be a [R, H, D] tensor")
    dt = _dtype_of(q)
    R, H, D = q.shape
    if not isinstance(k, torch.Tensor) or k.dim() != 2:
        raise PivotError("k must be a [Lk, D] tensor")
    Lk = k.shape[0]
    _expect(w, "w", (R, H), torch.float32)
    _expect(k, "k", (Lk, D), q.dtype)
    _scales(dt, q_scale, k_scale, (R,), (Lk,))
    _on_device(q=q, w=w, k=k, q_scale=q_scale, k_scale=k_scale)
    row_end = R if row_end is None else row_end
    S = torch.full((max(row_end - row_begin, 0), Lk), float("nan"), dtype=torch.float32,
                   device=q.device)
    _check(L.pivot_dbg_score_rows(_ptr(q), _ptr(q_scale), _ptr(w), _ptr(k), _ptr(k_scale), R, Lk,
                                  H, D, dt, row_begin, row_end, pos_mul, pos_add, _ptr(S), Lk,
                                  _stream(stream)))
    return S


def _decode_inputs(q, w, k_cache, cache_len, q_scale, k_scale):
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise PivotError("q must be a [B, g, H, D] tensor")
    dt = _dtype_of(q)
    B, g, H, D = q.shape
    if not isinstance(k_cache, torch.Tensor) or k_cache.dim() != 3:
        raise PivotError("k_cache must be a [B, Lmax, D] tensor")
    Lmax = k_cache.shape[1]
    _expect(w, "w", (B, g, H), torch.float32)
    _expect(k_cache, "k_cache", (B, Lmax, D), q.dtype)
    _expect(cache_len, "cache_len", (B,), torch.int32)
    _scales(dt, q_scale, k_scale, (B, g), (B, Lmax))
    return dt, B, g, H, D, Lmax


def indexer_decode(q, w, k_cache, cache_len, *, topk: int, C: int = 0, mode="refine",
                   q_scale=None, k_scale=None, out=None, workspace=None,
                   stream=None, window: int = 0, window_mode="shared", out_scores=None,
                   return_scores: bool = False):
    """One MTP decode step: q [B,g,H,D], w [B,g,H], k_cache [B,Lmax,D],
    cache_len [B] int32 (device); fp8 needs q_scale [B,g], k_scale [B,Lmax].
    Returns int32 [B, g, topk] ([B, g, topk + window] with a window); with
    return_scores (no window) also the float32 [B, g, topk] scores."""
    L = load()
    dt, B, g, H, D, Lmax = _decode_inputs(q, w, k_cache, cache_len, q_scale, k_scale)
    m = _mode(mode)
    if window < 0:
        raise PivotError("window must be >= 0")
    wm = _window_mode(window_mode)
    out = _out(out, "out", (B, g, topk + window), torch.int32, q.device)
    want = return_scores or out_scores is not None
    if want:
        if window:
            raise PivotError("scores are returned without a window only")
        out_scores = _out(out_scores, "out_scores", (B, g, topk), torch.float32, q.device)
    _on_device(q=q, w=w, k_cache=k_cache, cache_len=cache_len, q_scale=q_scale, k_scale=k_scale)
    ws = _workspace(L.pivot_decode_workspace_size(B, Lmax, H, D, g, topk, C, m, dt), q.device,
                    workspace)
    nbytes = ws.numel()
    if window:
        _check(L.pivot_indexer_decode_window(
            _ptr(q), _ptr(q_scale), _ptr(w), _ptr(k_cache), _ptr(k_scale), _ptr(cache_len), B,
            Lmax, H, D, g, topk, C, m, dt, window, wm, _ptr(out), _ptr(ws), nbytes, _stream(stream)))
    else:
        _check(L.pivot_indexer_decode(_ptr(q), _ptr(q_scale), _ptr(w), _ptr(k_cache),
                                      _ptr(k_scale), _ptr(cache_len), B, Lmax, H, D, g, topk, C, m,
                                      dt, _ptr(out), _ptr(out_scores), _ptr(ws), nbytes,
                                      _stream(stream)))
    return (out, out_scores) if want else out


def indexer_decode_noalloc(q, w, k_cache, cache_len, *, topk: int, C: int = 0, mode="refine",
                           q_scale=None, k_scale=None, out=None, out_scores=None, stream=None):
    """One MTP decode step through pivot_indexer_decode_noalloc: the library
    uses its own per-GPU scratch array and allocates nothing (arguments as
    for indexer_decode; out / out_scores may be passed in so that this
    function allocates nothing either).  Returns out, or (out, out_scores)
    when out_scores is given."""
    L = load()
    dt, B, g, H, D, Lmax = _decode_inputs(q, w, k_cache, cache_len, q_scale, k_scale)
    m = _mode(mode)
    out = _out(out, "out", (B, g, topk), torch.int32, q.device)
    if out_scores is not None:
        _expect(out_scores, "out_scores", (B, g, topk), torch.float32)
        _dev(out_scores, "out_scores")
    _on_device(q=q, w=w, k_cache=k_cache, cache_len=cache_len, q_scale=q_scale, k_scale=k_scale)
    _check(L.pivot_indexer_decode_noalloc(_ptr(q), _ptr(q_scale), _ptr(w), _ptr(k_cache), _ptr(k_scale),
                                          _ptr(cache_len), B, Lmax, H, D, g, topk, C, m, dt, _ptr(out),
                                          _ptr(out_scores), _stream(stream)))
    return out if out_scores is None else (out, out_scores)


def noalloc_scratch_bytes() -> int:
    return int(load().pivot_noalloc_scratch_bytes())


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
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise PivotError("q must be a [B, g, H, D] tensor")
    dt = _dtype_of(q)
    B, g, H, D = q.shape
    if not isinstance(k_pages, torch.Tensor) or k_pages.dim() != 3:
        raise PivotError("k_pages must be a [num_pages, page_size, D] tensor")
    if not isinstance(block_table, torch.Tensor) or block_table.dim() != 2:
        raise PivotError("block_table must be a [B, max_pages] tensor")
    num_pages, page_size = k_pages.shape[0], k_pages.shape[1]
    max_pages = block_table.shape[1]
    _expect(w, "w", (B, g, H), torch.float32)
    _expect(k_pages, "k_pages", (num_pages, page_size, D), q.dtype)
    _expect(block_table, "block_table", (B, max_pages), torch.int32)
    _expect(cache_len, "cache_len", (B,), torch.int32)
    _scales(dt, q_scale, k_scale, (B, g), (num_pages, page_size))
    _on_device(q=q, w=w, k_pages=k_pages, block_table=block_table, cache_len=cache_len,
               q_scale=q_scale, k_scale=k_scale)
    m = _mode(mode)
    wm = _window_mode(window_mode)
    out = _out(out, "out", (B, g, topk + window), torch.int32, q.device)
    ws = _workspace(L.pivot_decode_workspace_size(B, max_pages * page_size, H, D, g, topk, C, m, dt),
                    q.device, workspace)
    _check(L.pivot_indexer_decode_paged(
        _ptr(q), _ptr(q_scale), _ptr(w), _ptr(k_pages), _ptr(k_scale), num_pages, page_size,
        _ptr(block_table), max_pages, _ptr(cache_len), B, H, D, g, topk, C, m, dt, window, wm,
        _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def decode_candidates(q, w, k_cache, cache_len, *, topk: int, C: int = 0, mode="refine",
                      q_scale=None, k_scale=None, workspace=None, stream=None) -> torch.Tensor:
    """Every sequence's proxy top-m for one decode step: int32 [B, m]."""
    L = load()
    dt, B, g, H, D, Lmax = _decode_inputs(q, w, k_cache, cache_len, q_scale, k_scale)
    m = _mode(mode)
    _on_device(q=q, w=w, k_cache=k_cache, cache_len=cache_len, q_scale=q_scale, k_scale=k_scale)
    cand = torch.empty((B, C if m == REFINE else topk), dtype=torch.int32, device=q.device)
    ws = _workspace(L.pivot_decode_workspace_size(B, Lmax, H, D, g, topk, C, m, dt), q.device,
                    workspace)
    _check(L.pivot_decode_candidates(_ptr(q), _ptr(q_scale), _ptr(w), _ptr(k_cache),
                                     _ptr(k_scale), _ptr(cache_len), B, Lmax, H, D, g, topk, C,
                                     m, dt, _ptr(cand), _ptr(ws), ws.numel(), _stream(stream)))
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
    if not isinstance(q, torch.Tensor) or q.dim() != 3 or q.dtype != torch.bfloat16:
        raise PivotError("q must be a bf16 [R, Hq, d] tensor")
    R, Hq, d = q.shape
    if not isinstance(k, torch.Tensor) or not isinstance(v, torch.Tensor) or k.dim() != v.dim() \
            or k.dim() not in (2, 3):
        raise PivotError("k and v must both be [N, d] / [N, dv] or [B, S, d] / [B, S, dv] tensors")
    dv = v.shape[-1]
    _expect(k, "k", tuple(k.shape[:-1]) + (d,), torch.bfloat16)
    _expect(v, "v", tuple(k.shape[:-1]) + (dv,), torch.bfloat16)
    if not isinstance(idx, torch.Tensor) or idx.dim() != 2:
        raise PivotError("idx must be a [R, nidx] tensor")
    _expect(idx, "idx", (R, idx.shape[1]), torch.int32)
    if k.dim() == 2:
        stride, nkeys = 0, k.shape[0]
        rows_per_seq = R if rows_per_seq is None else rows_per_seq
    else:
        stride, nkeys = k.shape[1], k.shape[1]
        if rows_per_seq is None:
            raise PivotError("rows_per_seq is needed with per-sequence k/v")
        if (R + rows_per_seq - 1) // rows_per_seq > k.shape[0]:
            raise PivotError(f"{R} rows of {rows_per_seq} per sequence need more than {k.shape[0]} sequences")
    seq_len = nkeys if seq_len is None else seq_len
    if seq_len > nkeys:
        raise PivotError(f"seq_len={seq_len} exceeds the {nkeys} key rows per sequence")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    nidx = idx.shape[1]
    if out is not None:
        _expect(out, "out", (R, Hq, dv), torch.float32)
    _on_device(q=q, k=k, v=v, idx=idx)
    out = _out(out, "out", (R, Hq, dv), torch.float32, q.device)
    need = L.pivot_sparse_attention_workspace_size(R, Hq, dv, nidx)
    ws = _workspace(need, q.device, workspace) if need else None
    _check(L.pivot_sparse_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(idx), R, Hq, d, dv, nidx,
                                    rows_per_seq, stride, seq_len, float(scale), _ptr(out),
                                    _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))
    return out


def selftest_mfma_layout(device="cuda") -> torch.Tensor:
    """[3, 2, 64, 16] int32: row / column / pairing probes for bf16 and fp8 tiles."""
    L = load()
    out = torch.zeros((3, 2, 64, 16), dtype=torch.int32, device=device)
    _check(L.pivot_selftest_mfma_layout(_ptr(out), _stream(None)))
    return out


KERNEL_CLASSES = ("proxy_mean", "scan", "select", "refine_score", "member_select", "broadcast",
                  "decode_scan", "window", "attention", "layer_copy")


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
