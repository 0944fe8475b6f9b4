"""The C-ABI library loads, exports every function include/pivot.h declares, and
rejects bad arguments on the host before anything is launched.  CPU only: the
pointers below are never dereferenced because validation fails first."""
import ctypes as C
import os
import re

import pytest

import top_token_selection_pivot_amd as pv
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "pivot.h")

# the status set of include/pivot.h
(OK, ERR_NULL, ERR_SHAPE, ERR_PARAM, ERR_UNSUPPORTED, ERR_ALIGN, ERR_WORKSPACE, ERR_HIP,
 ERR_INTERNAL) = range(9)
FAKE = 0x100000  # aligned, never dereferenced


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pivot_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pv.library_path()):
        from top_token_selection_pivot_amd import build
        build.build(verbose=False)
    return pv.load()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert lib.pivot_version() >= 100
    for n in ("pivot_last_error_detail", "pivot_dbg_score_rows", "pivot_indexer", "pivot_indexer_decode"):
        assert n in names, n


def test_status_strings(lib):
    seen = set()
    for st in range(9):
        msg = lib.pivot_status_string(st).decode()
        assert msg and msg != "unknown status", st
        seen.add(msg)
    assert len(seen) == 9
    assert lib.pivot_status_string(99).decode() == "unknown status"


def _call(lib, **kw):
    a = dict(q=FAKE, qs=None, w=FAKE, k=FAKE, ks=None, L=2048, H=4, D=32, g=4, topk=64, C=256,
             mode=pv.REFINE, dtype=0, out=FAKE, scores=None, ws=FAKE, wsb=1 << 40, st=None)
    a.update(kw)
    return lib.pivot_indexer(a["q"], a["qs"], a["w"], a["k"], a["ks"], a["L"], a["H"], a["D"],
                             a["g"], a["topk"], a["C"], a["mode"], a["dtype"], a["out"], a["scores"],
                             a["ws"], a["wsb"], a["st"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), ERR_NULL),
    (dict(w=None), ERR_NULL),
    (dict(out=None), ERR_NULL),
    (dict(ws=None), ERR_NULL),
    (dict(dtype=1), ERR_NULL),               # fp8 without scales
    (dict(H=0), ERR_SHAPE),
    (dict(H=65), ERR_UNSUPPORTED),
    (dict(D=48), ERR_UNSUPPORTED),
    (dict(D=32, dtype=1, qs=FAKE, ks=FAKE), ERR_UNSUPPORTED),  # fp8 needs D in {64,128,256}
    (dict(L=0), ERR_SHAPE),
    (dict(g=0), ERR_PARAM),
    (dict(topk=0), ERR_PARAM),
    (dict(C=63), ERR_PARAM),                 # Refine needs C >= topk
    (dict(mode=7), ERR_PARAM),
    (dict(dtype=5), ERR_PARAM),
    (dict(q=FAKE + 8), ERR_ALIGN),
    (dict(k=FAKE + 4), ERR_ALIGN),
    (dict(w=FAKE + 2), ERR_ALIGN),
    (dict(ws=FAKE + 64), ERR_ALIGN),
    (dict(scores=FAKE + 2), ERR_ALIGN),
    (dict(wsb=1024), ERR_WORKSPACE),
    (dict(scores=FAKE, wsb=1024), ERR_WORKSPACE),  # scores are optional output only
])
def test_prefill_validation(lib, kw, status):
    assert _call(lib, **kw) == status
    assert lib.pivot_last_error_detail()  # a message is recorded


def test_reuse_ignores_C(lib):
    # Reuse does not use C, so C < topk is fine: the call only fails on the workspace here
    assert _call(lib, mode=pv.REUSE, C=0, wsb=16) == ERR_WORKSPACE


def test_decode_validation(lib):
    f = lib.pivot_indexer_decode
    base = [FAKE, None, FAKE, FAKE, None, FAKE, 32, 131072, 64, 128, 2, 2048, 4096, pv.REFINE, 0,
            FAKE, None, FAKE, 1 << 40, None]
    def call(**kw):
        a = list(base)
        idx = dict(q=0, w=2, k=3, cl=5, B=6, Lmax=7, H=8, D=9, g=10, topk=11, C=12, mode=13,
                   dtype=14, out=15, scores=16, ws=17, wsb=18)
        for k_, v in kw.items():
            a[idx[k_]] = v
        return f(*a)
    assert call(cl=None) == ERR_NULL
    assert call(B=0) == ERR_SHAPE
    assert call(g=200000) == ERR_PARAM
    assert call(C=100) == ERR_PARAM
    assert call(wsb=100) == ERR_WORKSPACE
    assert call(dtype=1) == ERR_NULL
    assert call(H=65) == ERR_UNSUPPORTED
    assert call(scores=FAKE + 1) == ERR_ALIGN
    assert call(scores=FAKE, wsb=100) == ERR_WORKSPACE


def test_score_rows_validation(lib):
    def f(**kw):
        a = dict(q=FAKE, qs=None, w=FAKE, k=FAKE, ks=None, R=64, Lk=4096, H=64, D=128, dt=0, rb=0, re=64,
                 pm=1, pa=0, S=FAKE, ld=4096)
        a.update(kw)
        return lib.pivot_dbg_score_rows(a["q"], a["qs"], a["w"], a["k"], a["ks"], a["R"], a["Lk"], a["H"],
                                        a["D"], a["dt"], a["rb"], a["re"], a["pm"], a["pa"], a["S"], a["ld"],
                                        None)
    assert f(q=None) == ERR_NULL
    assert f(S=None) == ERR_NULL
    assert f(dt=1) == ERR_NULL  # fp8 needs scales
    assert f(R=0) == ERR_SHAPE
    assert f(re=65) == ERR_SHAPE
    assert f(rb=10, re=5) == ERR_SHAPE
    assert f(H=65) == ERR_UNSUPPORTED
    assert f(D=96) == ERR_UNSUPPORTED
    assert f(pm=-1) == ERR_PARAM
    assert f(ld=63) == ERR_PARAM  # the last row sees keys 0..63
    assert f(S=FAKE + 2) == ERR_ALIGN
    assert f(rb=5, re=5) == OK    # no rows: nothing to launch



def test_workspace_sizes(lib):
    # minimum <= preferred; both grow with L; Reuse needs less than Refine
    for mode in (pv.DENSE, pv.REUSE, pv.REFINE):
        mn = lib.pivot_workspace_min_size(131072, 64, 128, 8, 2048, 4096, mode, 0)
        pf = lib.pivot_workspace_size(131072, 64, 128, 8, 2048, 4096, mode, 0)
        assert 0 < mn <= pf
    assert lib.pivot_workspace_size(0, 64, 128, 8, 2048, 4096, pv.REFINE, 0) == 0
    assert (lib.pivot_workspace_size(16384, 64, 128, 8, 2048, 4096, pv.REUSE, 0)
            < lib.pivot_workspace_size(16384, 64, 128, 8, 2048, 4096, pv.REFINE, 0))
    assert lib.pivot_decode_workspace_size(32, 131072, 64, 128, 2, 2048, 4096, pv.REFINE, 1) > 32 * 131072 * 4


def test_python_binding_fails_loudly_without_device():
    import torch
    q = torch.zeros((16, 4, 32), dtype=torch.bfloat16)
    with pytest.raises(pv.PivotError):
        pv.indexer(q, torch.zeros((16, 4)), torch.zeros((16, 32), dtype=torch.bfloat16), g=4,
                   topk=4, C=8)


def test_window_validation(lib):
    # the window entry points check window and window_mode before anything runs
    def pre(window, wmode, **kw):
        a = dict(q=FAKE, w=FAKE, k=FAKE, out=FAKE, ws=FAKE, wsb=1 << 40)
        a.update(kw)
        return lib.pivot_indexer_window(a["q"], None, a["w"], a["k"], None, 2048, 4, 32, 4, 64,
                                        256, pv.REFINE, 0, window, wmode, a["out"], a["ws"],
                                        a["wsb"], None)

    def dec(window, wmode, **kw):
        a = dict(out=FAKE, wsb=1 << 40)
        a.update(kw)
        return lib.pivot_indexer_decode_window(FAKE, None, FAKE, FAKE, None, FAKE, 32, 131072, 64,
                                               128, 2, 2048, 4096, pv.REFINE, 0, window, wmode,
                                               a["out"], FAKE, a["wsb"], None)
    for f in (pre, dec):
        assert f(-1, 0) == ERR_PARAM
        assert f(3, 2) == ERR_PARAM
        assert f(3, -1) == ERR_PARAM
        assert f(1 << 30, 1) == ERR_PARAM
        assert f(3, 0, out=None) == ERR_NULL
        assert f(3, 1, wsb=100) == ERR_WORKSPACE  # valid window: fails only on the workspace


def test_sparse_attention_validation(lib):
    def f(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, idx=FAKE, R=64, Hq=64, d=128, dv=128, nidx=2048, rps=2,
                 stride=131072, seq_len=131072, scale=0.088, out=FAKE, ws=FAKE, wsb=100)
        a.update(kw)
        return lib.pivot_sparse_attention(a["q"], a["k"], a["v"], a["idx"], a["R"], a["Hq"], a["d"],
                                          a["dv"], a["nidx"], a["rps"], a["stride"], a["seq_len"],
                                          a["scale"], a["out"], a["ws"], a["wsb"], None)
    assert f(q=None) == ERR_NULL
    assert f(Hq=48) == ERR_UNSUPPORTED
    assert f(d=64) == ERR_UNSUPPORTED
    assert f(R=0) == ERR_SHAPE
    assert f(rps=0) == ERR_PARAM
    assert f(stride=100) == ERR_PARAM          # sequences would overlap
    assert f(scale=0.0) == ERR_PARAM
    assert f(out=FAKE + 4) == ERR_ALIGN
    assert f(seq_len=1 << 23, stride=1 << 23) == ERR_SHAPE  # 2^23 rows of 256 bytes: 2 GiB
    assert f(seq_len=(1 << 23) - 1, stride=1 << 23) == ERR_WORKSPACE  # just below 2 GiB passes
    assert f() == ERR_WORKSPACE                 # 64 rows: chunks merged through the workspace
    assert lib.pivot_sparse_attention_workspace_size(64, 64, 128, 2048) > 0
    assert lib.pivot_sparse_attention_workspace_size(4096, 64, 128, 2048) == 0  # one chunk per row


def test_varlen_validation(lib):
    import ctypes
    import numpy as np

    def f(cu, **kw):
        a = dict(q=FAKE, w=FAKE, k=FAKE, out=FAKE, wsb=1 << 40, mode=pv.REFINE)
        a.update(kw)
        arr = None if cu is None else np.ascontiguousarray(cu, np.int64)
        return lib.pivot_indexer_varlen(a["q"], None, a["w"], a["k"], None,
                                        None if arr is None else arr.ctypes.data, 0 if cu is None else len(cu) - 1,
                                        4, 32, 4, 64, 256, a["mode"], 0, 0, 0, a["out"], FAKE, a["wsb"], None)
    assert f(None) == ERR_NULL
    assert f([0]) == ERR_SHAPE                   # no sequence
    assert f([1, 5]) == ERR_PARAM                # must start at 0
    assert f([0, 9, 5]) == ERR_PARAM             # decreasing
    assert f([0, 9, 20], out=None) == ERR_NULL
    assert f([0, 9, 20], mode=9) == ERR_PARAM
    assert f([0, 2048, 4096], wsb=1000) == ERR_WORKSPACE
    cu = np.array([0, 100, 100, 3000], np.int64)
    big = lib.pivot_varlen_workspace_size(cu.ctypes.data, 3, 4, 32, 4, 64, 256, pv.REFINE, 0)
    one = lib.pivot_workspace_size(2900, 4, 32, 4, 64, 256, pv.REFINE, 0)
    assert big == 2 * ((one + 255) // 256 * 256)  # a slice per non-empty sequence (at most four)
    cu8 = np.arange(9, dtype=np.int64) * 100
    assert lib.pivot_varlen_workspace_size(cu8.ctypes.data, 8, 4, 32, 4, 64, 256, pv.REFINE, 0) == 4 * (
        (lib.pivot_workspace_size(100, 4, 32, 4, 64, 256, pv.REFINE, 0) + 255) // 256 * 256)


def test_paged_decode_validation(lib):
    # the paged decode entry checks the pool and the block table before
    # anything runs; with valid pages it fails only on the workspace
    def f(**kw):
        a = dict(num_pages=2100, page_size=64, bt=FAKE, max_pages=2048, D=128, dt=1, wsb=100,
                 out=FAKE, ks=FAKE)
        a.update(kw)
        return lib.pivot_indexer_decode_paged(FAKE, FAKE, FAKE, FAKE, a["ks"], a["num_pages"],
                                              a["page_size"], a["bt"], a["max_pages"], FAKE, 32, 64,
                                              a["D"], 2, 2048, 4096, pv.REFINE, a["dt"], 0, 0,
                                              a["out"], FAKE, a["wsb"], None)
    assert f() == ERR_WORKSPACE
    assert f(page_size=1024, max_pages=128) == ERR_WORKSPACE
    assert f(bt=None) == ERR_NULL
    assert f(out=None) == ERR_NULL
    assert f(ks=None) == ERR_NULL  # fp8 needs the pool's scales
    assert f(bt=FAKE + 2) == ERR_ALIGN
    for ps in (0, 32, 96, 1 << 21):
        assert f(page_size=ps) == ERR_PARAM, ps
    assert f(num_pages=0) == ERR_SHAPE
    assert f(max_pages=0) == ERR_SHAPE
    # the pool must stay below 4 GiB of key codes: 2^26 keys of 64 bytes is 4 GiB
    assert f(num_pages=1 << 20, page_size=64, D=64) == ERR_SHAPE
    assert f(num_pages=(1 << 20) - 1, page_size=64, D=64) == ERR_WORKSPACE


def test_layers_validation(lib):
    import numpy as np
    P = lambda n, v=FAKE: np.full(n, v, np.uint64)

    def f(full, **kw):
        fl = np.ascontiguousarray(full, np.int32)
        n = len(full)
        a = dict(q=P(n), w=P(n), k=P(n), out=P(n), wsb=1 << 40, C=256)
        a.update(kw)
        arr = {k_: (None if v is None else v.ctypes.data) for k_, v in a.items() if k_ in ("q", "w", "k", "out")}
        return lib.pivot_indexer_layers(n, fl.ctypes.data, arr["q"], None, arr["w"], arr["k"], None, 2048, 4, 32, 4,
                                        64, a["C"], pv.REFINE, 0, arr["out"], FAKE, a["wsb"], None)
    assert f([0, 1]) == ERR_PARAM          # layer 0 must run its indexer
    assert f([1, 0], out=None) == ERR_NULL
    assert f([1, 0], q=None) == ERR_NULL
    assert f([1, 1], out=np.array([FAKE, 0], np.uint64)) == ERR_NULL
    assert f([1, 1], C=10) == ERR_PARAM    # a full layer's own checks
    assert b"layer 0" in lib.pivot_last_error_detail()
    assert f([1, 0, 1], wsb=100) == ERR_WORKSPACE
    assert lib.pivot_indexer_layers(0, None, None, None, None, None, None, 1, 1, 32, 1, 1, 1, 0, 0, None, None, 0,
                                    None) == ERR_SHAPE
