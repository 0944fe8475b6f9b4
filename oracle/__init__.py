"""CPU oracle of the PIVOT query-group indexer (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg; never by the product package.  The arithmetic
lives in pivot_oracle.c (plain single-threaded C, double accumulation); this
file only marshals numpy arrays.

Pinned functions (see tests/test_oracle_*.py): codecs, score, top-m, dense,
proxy, Reuse, Refine, decode grouping, sliding-window union and exclusion, the
paged-cache view, cross-layer index reuse (its layer bookkeeping is here, in
Python; every full layer is the C oracle's indexer).  Parity on realistic float inputs is
pinned only through invariants and the closed-form/worked examples.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# PIVOT_ORACLE_LIB names a prebuilt variant of the same source (the planted-
# mistake test builds such variants to show that the pins catch them)
_VARIANT = os.environ.get("PIVOT_ORACLE_LIB")
_LIB_PATH = _VARIANT or os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "pivot_oracle.c")
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-Wall"]

BF16, FP8 = 0, 1
DENSE, REUSE, REFINE = 0, 1, 2
MODES = {"dense": DENSE, "reuse": REUSE, "refine": REFINE}


def build(force: bool = False) -> str:
    """Compile pivot_oracle.c with gcc (plain -O2, IEEE binary32/binary64, no
    contraction of multiply-adds, single-threaded)."""
    if _VARIANT:
        return _LIB_PATH
    if force or not os.path.exists(_LIB_PATH):
        subprocess.run(["gcc", *CFLAGS, "-o", _LIB_PATH, _SRC, "-lm"], check=True)
    return _LIB_PATH


class _View(C.Structure):
    _fields_ = [("H", C.c_int), ("D", C.c_int), ("dtype", C.c_int),
                ("q", C.c_void_p), ("q_scale", C.c_void_p), ("w", C.c_void_p),
                ("k", C.c_void_p), ("k_scale", C.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = C.CDLL(_LIB_PATH)
        i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
        f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
        L.orc_bf16_value.restype = C.c_double
        L.orc_bf16_value.argtypes = [C.c_uint16]
        L.orc_e4m3_value.restype = C.c_double
        L.orc_e4m3_value.argtypes = [C.c_uint8]
        L.orc_bf16_from_f32.restype = C.c_uint16
        L.orc_bf16_from_f32.argtypes = [C.c_float]
        L.orc_e4m3_from_f32.restype = C.c_uint8
        L.orc_e4m3_from_f32.argtypes = [C.c_float]
        L.orc_topk.argtypes = [C.c_int, i32p, f64p, C.c_int, i32p]
        L.orc_proxy.argtypes = [C.POINTER(_View), C.c_int, C.c_int, C.c_void_p,
                                C.POINTER(C.c_float), C.c_void_p]
        L.orc_dense_rows.argtypes = [C.POINTER(_View), i32p, C.c_int, C.c_int, i32p]
        L.orc_group.argtypes = [C.POINTER(_View), C.c_int, C.c_int, C.c_int, C.c_int, C.c_int,
                                C.c_int, i32p, C.c_void_p, C.c_void_p]
        L.orc_prefill_groups.argtypes = [C.POINTER(_View), C.c_int, C.c_int, C.c_int, C.c_int,
                                         C.c_int, i32p, C.c_int, i32p, C.c_void_p]
        L.orc_dense_rows_ex.argtypes = [C.POINTER(_View), i32p, C.c_int, C.c_int, C.c_int, i32p]
        L.orc_group_ex.argtypes = [C.POINTER(_View), C.c_int, C.c_int, C.c_int, C.c_int, C.c_int,
                                   C.c_int, C.c_int, i32p, C.c_void_p, C.c_void_p]
        L.orc_prefill_groups_ex.argtypes = [C.POINTER(_View), C.c_int, C.c_int, C.c_int, C.c_int,
                                            C.c_int, C.c_int, i32p, C.c_int, i32p, C.c_void_p]
        L.orc_window_union.argtypes = [i32p, C.c_int, C.c_int, C.c_int, i32p]
        u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
        L.orc_sparse_attention.argtypes = [u16p, u16p, u16p, i32p] + [C.c_int] * 6 + [
            C.c_long, C.c_int, C.c_double, f64p]
        L.orc_score_row.argtypes = [C.POINTER(_View), C.c_int, C.c_int, f64p]
        L.orc_score_pairs.argtypes = [C.POINTER(_View), i32p, i32p, C.c_int, f64p]
        L.orc_score_list.argtypes = [C.POINTER(_View), C.c_int, i32p, C.c_int, f64p]
        L.orc_init.argtypes = []
        L.orc_init()  # tables filled once, before any thread uses the oracle
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


class View:
    """Keeps the numpy arrays alive and exposes them as an orc_view.

    q [R,H,D] codes, q_scale [R] or None, w [R,H], k [N,D] codes, k_scale [N] or None."""

    def __init__(self, dtype, q, q_scale, w, k, k_scale):
        self.dtype = BF16 if dtype in ("bf16", BF16) else FP8
        code_t = np.uint16 if self.dtype == BF16 else np.uint8
        self.q = np.ascontiguousarray(q, dtype=code_t)
        self.k = np.ascontiguousarray(k, dtype=code_t)
        self.w = np.ascontiguousarray(w, dtype=np.float32)
        self.q_scale = None if q_scale is None else np.ascontiguousarray(q_scale, np.float32)
        self.k_scale = None if k_scale is None else np.ascontiguousarray(k_scale, np.float32)
        if self.dtype == FP8 and (self.q_scale is None or self.k_scale is None):
            raise ValueError("fp8 views need q_scale and k_scale")
        self.H, self.D = int(self.q.shape[-2]), int(self.q.shape[-1])
        self.c = _View(self.H, self.D, self.dtype, _ptr(self.q), _ptr(self.q_scale),
                       _ptr(self.w), _ptr(self.k), _ptr(self.k_scale))

    @classmethod
    def of(cls, inp):
        return cls(inp.dtype, inp.q, inp.q_scale, inp.w, inp.k, inp.k_scale)


def bf16_value(code):
    return lib().orc_bf16_value(int(code))


def e4m3_value(code):
    return lib().orc_e4m3_value(int(code))


def bf16_from_f32(x):
    return lib().orc_bf16_from_f32(float(x))


def e4m3_from_f32(x):
    return lib().orc_e4m3_from_f32(float(x))


def topk(scores, m, pos=None):
    scores = np.ascontiguousarray(scores, np.float64)
    n = scores.shape[0]
    pos = np.arange(n, dtype=np.int32) if pos is None else np.ascontiguousarray(pos, np.int32)
    out = np.empty(m, np.int32)
    lib().orc_topk(n, pos, scores, m, out)
    return out


def proxy(view: View, row0: int, n: int):
    code_t = np.uint16 if view.dtype == BF16 else np.uint8
    codes = np.empty((view.H, view.D), code_t)
    wbar = np.empty(view.H, np.float32)
    s = C.c_float(0.0)
    lib().orc_proxy(C.byref(view.c), row0, n, codes.ctypes.data, C.byref(s), wbar.ctypes.data)
    return codes, np.float32(s.value), wbar


def dense_rows(view: View, rows, topk_: int, excl: int = 0):
    """Dense top-k of the listed rows; excl > 0: row t chooses among 0..t-excl."""
    rows = np.ascontiguousarray(rows, np.int32)
    out = np.empty((rows.shape[0], topk_), np.int32)
    if excl:
        lib().orc_dense_rows_ex(C.byref(view.c), rows, rows.shape[0], topk_, excl, out)
    else:
        lib().orc_dense_rows(C.byref(view.c), rows, rows.shape[0], topk_, out)
    return out


def group(view: View, row0: int, pos0: int, n: int, topk_: int, C_: int, mode, excl: int = 0):
    """One group; returns (out [n,topk], cand [m] or None, proxy scores [pos0+n-excl]).
    excl > 0: the window is excluded, member t chooses among 0..t-excl."""
    mode = MODES.get(mode, mode)
    out = np.empty((n, topk_), np.int32)
    m = C_ if mode == REFINE else topk_
    cand = np.empty(m, np.int32) if mode != DENSE else None
    psc = np.empty(max(pos0 + n - excl, 1), np.float64) if mode != DENSE else None
    if excl:
        lib().orc_group_ex(C.byref(view.c), row0, pos0, n, topk_, C_, mode, excl, out,
                           _ptr(cand), _ptr(psc))
    else:
        lib().orc_group(C.byref(view.c), row0, pos0, n, topk_, C_, mode, out,
                        _ptr(cand), _ptr(psc))
    if psc is not None:
        psc = psc[:max(pos0 + n - excl, 0)]
    return out, cand, psc


def prefill_groups(view: View, L: int, g: int, topk_: int, C_: int, mode, groups,
                   excl: int = 0):
    """Rows of the listed prefill groups (packed) and their candidate lists."""
    mode = MODES.get(mode, mode)
    groups = np.ascontiguousarray(groups, np.int32)
    nrows = int(sum(min(g, L - int(j) * g) for j in groups))
    out = np.empty((nrows, topk_), np.int32)
    m = C_ if mode == REFINE else topk_
    cand = np.empty((groups.shape[0], m), np.int32) if mode != DENSE else None
    if excl:
        lib().orc_prefill_groups_ex(C.byref(view.c), L, g, topk_, C_, mode, excl, groups,
                                    groups.shape[0], out, _ptr(cand))
    else:
        lib().orc_prefill_groups(C.byref(view.c), L, g, topk_, C_, mode, groups,
                                 groups.shape[0], out, _ptr(cand))
    return out, cand


def window_union(sel, positions, W: int):
    """Sliding window of size W added to selections ([TUT] section on combining
    the recent window with the selected positions, Figure 3): sel [rows, k]
    ascending, -1 padded; positions [rows] the queries' positions.  Returns
    [rows, k + W]: the union, ascending, each position once, -1 padded."""
    sel = np.ascontiguousarray(sel, np.int32)
    rows, k = sel.shape
    out = np.empty((rows, k + W), np.int32)
    for r in range(rows):
        o = np.empty(k + W, np.int32)
        lib().orc_window_union(np.ascontiguousarray(sel[r]), k, int(positions[r]), W, o)
        out[r] = o
    return out


WINDOW_SHARED, WINDOW_EXCLUDED = 0, 1
WINDOW_MODES = {"shared": WINDOW_SHARED, "excluded": WINDOW_EXCLUDED}


def prefill_window(view: View, L: int, g: int, topk_: int, C_: int, mode, groups, W: int,
                   wmode):
    """Listed prefill groups' rows with a sliding window of size W: "shared"
    (the window's positions stay candidates; union with the selection) or
    "excluded" (query t chooses among 0..t-W, then the window is added)."""
    wmode = WINDOW_MODES.get(wmode, wmode)
    sel, cand = prefill_groups(view, L, g, topk_, C_, mode, groups,
                               excl=W if wmode == WINDOW_EXCLUDED else 0)
    return window_union(sel, group_rows(L, g, groups), W), cand


def decode_seq_window(dec, b: int, topk_: int, C_: int, mode, W: int, wmode):
    """decode_seq with a sliding window of size W (see prefill_window)."""
    wmode = WINDOW_MODES.get(wmode, wmode)
    n = int(dec.cache_len[b])
    sel, cand, _ = group(decode_view(dec, b), 0, n - dec.g, dec.g, topk_, C_, mode,
                         excl=W if wmode == WINDOW_EXCLUDED else 0)
    return window_union(sel, np.arange(n - dec.g, n), W), cand


def _reuse_sources(full):
    """For every layer, the layer whose index rows it uses: itself when it runs
    its indexer, else the nearest such layer before it."""
    src, last = [], None
    for l, f in enumerate(full):
        if f:
            last = l
        elif last is None:
            raise ValueError("layer 0 must run its indexer")
        src.append(last)
    return src


def index_cache_prefill(views, L: int, g: int, topk_: int, C_: int, mode, full, groups):
    """Cross-layer index reuse stacked on the indexer (molayo1419.me "PIVOT
    explained", Try it now and Sources: IndexCache, "Accelerating Sparse
    Attention via Cross-Layer Index Reuse"; only the title is on the pages).
    Reading: layer l with full[l] runs the indexer (prefill_groups, any mode)
    on its own inputs views[l]; any other layer takes the rows of the nearest
    full layer before it.  Returns the listed groups' rows for every layer."""
    src = _reuse_sources(full)
    rows = {}
    for l, s in enumerate(src):
        if s == l:
            rows[l], _ = prefill_groups(views[l], L, g, topk_, C_, mode, groups)
    return [rows[s].copy() for s in src]


def index_cache_decode(decs, b: int, topk_: int, C_: int, mode, full):
    """The same reuse over decode steps: decs[l] is layer l's decode step
    (sharing the cache lengths); returns sequence b's [g, topk] rows per layer."""
    src = _reuse_sources(full)
    rows = {}
    for l, s in enumerate(src):
        if s == l:
            rows[l], _, _ = decode_seq(decs[l], b, topk_, C_, mode)
    return [rows[s].copy() for s in src]


def group_rows(L: int, g: int, groups):
    """Query positions covered by the listed groups, in the packed order."""
    return np.concatenate([np.arange(int(j) * g, min(L, int(j) * g + g)) for j in groups]
                          ).astype(np.int32)


def score_row(view: View, row: int, n: int):
    out = np.empty(n, np.float64)
    lib().orc_score_row(C.byref(view.c), row, n, out)
    return out


def score_list(view: View, row: int, keys):
    """Scores of query row `row` against the listed keys."""
    keys = np.ascontiguousarray(keys, np.int32)
    out = np.empty(keys.shape[0], np.float64)
    if keys.shape[0]:
        lib().orc_score_list(C.byref(view.c), int(row), keys, keys.shape[0], out)
    return out


def score_pairs(view: View, rows, keys):
    rows = np.ascontiguousarray(rows, np.int32)
    keys = np.ascontiguousarray(keys, np.int32)
    out = np.empty(rows.shape[0], np.float64)
    lib().orc_score_pairs(C.byref(view.c), rows, keys, rows.shape[0], out)
    return out


def decode_view(dec, b: int) -> View:
    """View of sequence b of a decode step: its g query rows and its key cache."""
    qs = None if dec.q_scale is None else dec.q_scale[b]
    ks = None if dec.k_scale is None else dec.k_scale[b]
    return View(dec.dtype, dec.q[b], qs, dec.w[b], dec.k[b], ks)


def decode_seq(dec, b: int, topk_: int, C_: int, mode):
    """Decode grouping (arXiv:2607.24593 abstract: in decode a group is the set
    of queries one MTP step produces): members at positions n_b-g..n_b-1, the
    shared scan covers the whole cache [0, n_b)."""
    n = int(dec.cache_len[b])
    return group(decode_view(dec, b), 0, n - dec.g, dec.g, topk_, C_, mode)


def paged_keys(k_pages, k_scale_pages, block_table, cache_len, Lmax: int):
    """The contiguous key cache [B, Lmax, D] (scales [B, Lmax], or None) that a
    paged cache stands for.  Position p < cache_len[b] of sequence b is row
    p % page_size of page block_table[b, p // page_size]; a page id outside
    [0, num_pages) stands for zero keys with zero scales; positions past
    cache_len[b] are zero.  Paging is a storage layout, not part of the
    method: a decode step over a paged cache is defined as the step over this
    contiguous cache (decode grouping as in decode_seq)."""
    k_pages = np.asarray(k_pages)
    num_pages, page_size, D = k_pages.shape
    B = block_table.shape[0]
    k = np.zeros((B, Lmax, D), k_pages.dtype)
    ks = None if k_scale_pages is None else np.zeros((B, Lmax), np.float32)
    for b in range(B):
        for p in range(int(cache_len[b])):
            pg = int(block_table[b, p // page_size])
            if 0 <= pg < num_pages:
                k[b, p] = k_pages[pg, p % page_size]
                if ks is not None:
                    ks[b, p] = k_scale_pages[pg, p % page_size]
    return k, ks


def sparse_attention(q, k, v, idx, rows_per_seq=None, seq_len=None, scale=None):
    """Sparse main attention over the selected positions ([TUT] text after
    Figure 1), multi-query layout, in double.  q [R,Hq,d] bf16 codes; k [N,d] or
    [B,S,d] and v [N,dv] or [B,S,dv] bf16 codes; idx [R,nidx].  Row r reads
    sequence r // rows_per_seq (default: one sequence).  Returns [R,Hq,dv]."""
    q = np.ascontiguousarray(q, np.uint16)
    idx = np.ascontiguousarray(idx, np.int32)
    R, Hq, d = q.shape
    dv = v.shape[-1]
    if k.ndim == 2:
        stride, nkeys = 0, k.shape[0]
        rows_per_seq = R if rows_per_seq is None else rows_per_seq
    else:
        stride, nkeys = k.shape[1], k.shape[1]
    k = np.ascontiguousarray(k, np.uint16).reshape(-1, d)
    v = np.ascontiguousarray(v, np.uint16).reshape(-1, dv)
    seq_len = nkeys if seq_len is None else seq_len
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    out = np.empty((R, Hq, dv), np.float64)
    lib().orc_sparse_attention(q, k, v, idx, R, Hq, d, dv, idx.shape[1], rows_per_seq, stride,
                               seq_len, float(scale), out)
    return out
