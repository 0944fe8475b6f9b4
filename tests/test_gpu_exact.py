"""GPU parity on integer-valued inputs: every binary32 sum is exact there, so the
HIP path must reproduce the oracle's indices bit for bit.  Covers the
matrix-core layout probe, the pages' worked example, the tiny prefill workload
(L=2048, H=4, D=32, g=4, topk=64, C=256), proxy bits, candidate sets, edge
cases (ragged groups, short rows, tiny and maximal shapes, chunked passes)
and the decode grouping."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
import top_token_selection_pivot_amd as pv
from conftest import GOLDEN
import parity
from parity import to_device

pytestmark = pytest.mark.gpu


def _run(inp, mode, g, topk, C, **kw):
    d = to_device(inp)
    out = pv.indexer(d["q"], d["w"], d["k"], g=g, topk=topk, C=C, mode=mode,
                     q_scale=d["q_scale"], k_scale=d["k_scale"], **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _oracle_all(inp, mode, g, topk, C):
    v = oracle.View.of(inp)
    if mode == "dense":
        return oracle.dense_rows(v, np.arange(inp.L), topk)
    G = (inp.L + g - 1) // g
    rows, _ = oracle.prefill_groups(v, inp.L, g, topk, C, mode, np.arange(G))
    return rows


def test_mfma_layout_selftest():
    print("case: matrix-core layout probe", flush=True)
    out = pv.selftest_mfma_layout().cpu().numpy()  # [probe][fmt][lane][acc]
    lane = np.arange(64)[:, None]
    i = np.arange(16)[None, :]
    rows = 8 * (i // 4) + 4 * (lane // 32) + (i % 4)
    cols = np.broadcast_to(lane % 32, (64, 16))
    for f in (0, 1):
        assert np.array_equal(out[0, f], rows), f"row layout, format {f}"
        assert np.array_equal(out[1, f], cols), f"column layout, format {f}"
        assert np.all(out[2, f] == 1), f"k-slice pairing, format {f}"


def _pad_view(q, w, k, H=1, D=32):
    """Zero-pad the pages' 2-d example to D=32 (zero padding leaves every score
    unchanged)."""
    L = q.shape[0]
    qp = np.zeros((L, H, D), np.float32)
    qp[:, :q.shape[1], :q.shape[2]] = q
    kp = np.zeros((L, D), np.float32)
    kp[:, :k.shape[1]] = k
    return synth.PrefillInputs("bf16", L, H, D, synth.encode_bf16(qp), None,
                               np.asarray(w, np.float32), synth.encode_bf16(kp), None)


def test_worked_example_fig1():
    print("case: worked example (Figure 1), dense top-3", flush=True)
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_fig1.json")))
    a = ex["keys_first_component"]
    b = ex["keys_second_component_p0_to_p6"] + [ex["key_p7_second_component"]]
    q = np.zeros((8, 1, 2), np.float32)
    q[:, 0] = [1, 0]
    q[6, 0] = ex["query_p6"]
    q[7, 0] = ex["query_p7"]
    inp = _pad_view(q, np.ones((8, 1)), np.stack([a, b], 1))
    out = _run(inp, "dense", 1, 3, 3)
    assert out[7].tolist() == ex["top3_p7"]
    assert out[6].tolist() == ex["top3_p6"]


def test_derived_pivot_example():
    print("case: derived PIVOT example, g=2", flush=True)
    ex = json.load(open(os.path.join(GOLDEN, "derived_pivot_example.json")))
    q = np.zeros((8, 1, 2), np.float32)
    q[:6, 0] = [[1, 0], [0, 1]] * 3
    q[6, 0] = ex["q6"]
    q[7, 0] = ex["q7"]
    inp = _pad_view(q, np.ones((8, 1)), np.stack([ex["a"], ex["b"]], 1))
    out = _run(inp, "reuse", 2, 3, 3)
    assert out[6].tolist() == ex["reuse_k3"]["member6"]
    assert out[7].tolist() == ex["reuse_k3"]["member7"]
    out = _run(inp, "refine", 2, 3, 4)
    assert out[6].tolist() == ex["refine_k3_C4"]["member6"]
    assert out[7].tolist() == ex["refine_k3_C4"]["member7"]
    out = _run(inp, "refine", 2, 3, 8)
    assert out[6].tolist() == ex["refine_k3_C8"]["member6"]
    assert out[7].tolist() == ex["refine_k3_C8"]["member7"]
    # every row, against the oracle
    for mode, C_ in (("reuse", 3), ("refine", 4), ("refine", 8), ("dense", 3)):
        assert np.array_equal(_run(inp, mode, 2, 3, C_), _oracle_all(inp, mode, 2, 3, C_))


@pytest.fixture(scope="module")
def tiny():
    return synth.make("tiny_prefill_2k")


@pytest.mark.parametrize("mode", ["dense", "reuse", "refine"])
def test_tiny_prefill_bit_exact(tiny, mode):
    print(f"case: tiny prefill L=2048 H=4 D=32 g=4 k=64 C=256 {mode}", flush=True)
    got = _run(tiny, mode, 4, 64, 256)
    ref = _oracle_all(tiny, mode, 4, 64, 256)
    assert np.array_equal(got, ref)


def test_tiny_proxy_bits_and_candidates(tiny):
    print("case: tiny prefill proxy bits and candidate sets", flush=True)
    d = to_device(tiny)
    v = oracle.View.of(tiny)
    for g in (4, 3, 16):
        qbar, qs, wbar = pv.proxy_mean(d["q"], d["w"], g)
        qbar = qbar.view(torch.int16).cpu().numpy().view(np.uint16)
        qs, wbar = qs.cpu().numpy(), wbar.cpu().numpy()
        for j in list(range(0, 2048 // g, 37)) + [(2048 + g - 1) // g - 1]:
            n = min(g, 2048 - j * g)
            c, s, wb = oracle.proxy(v, j * g, n)
            assert np.array_equal(qbar[j], c) and qs[j] == s and np.array_equal(wbar[j], wb)
    for mode, m in (("refine", 256), ("reuse", 64)):
        cand = pv.candidates(d["q"], d["w"], d["k"], g=4, topk=64, C=256, mode=mode).cpu().numpy()
        _, ref = oracle.prefill_groups(v, 2048, 4, 64, 256, mode, np.arange(512))
        assert np.array_equal(cand, ref)


@pytest.mark.parametrize("mode", ["dense", "reuse", "refine"])
def test_tiny_scores_exact(tiny, mode):
    """The scores returned with the selection are the exact scores on the tiny
    workload (every binary32 sum is exact there): the member's own score for
    dense and Refine, the proxy's score for Reuse; NaN past the selection."""
    print(f"case: tiny prefill scores, {mode}", flush=True)
    d = to_device(tiny)
    out, sc = pv.indexer(d["q"], d["w"], d["k"], g=4, topk=64, C=256, mode=mode, return_scores=True)
    torch.cuda.synchronize()
    out, sc = out.cpu().numpy(), sc.cpu().numpy()
    assert np.array_equal(out, _oracle_all(tiny, mode, 4, 64, 256))
    v = oracle.View.of(tiny)
    for j in range(2048 // 4):
        psc = oracle.group(v, 4 * j, 4 * j, 4, 64, 256, "reuse")[2] if mode == "reuse" else None
        for t in range(4 * j, 4 * j + 4):
            sel = out[t][out[t] >= 0]
            ref = psc[sel] if mode == "reuse" else oracle.score_list(v, t, sel)
            assert np.array_equal(sc[t][:len(sel)].astype(np.float64), ref), t
            assert np.all(np.isnan(sc[t][len(sel):])), t


def test_tiny_score_rows_exact(tiny):
    """The score-row export: dense rows and proxy rows of the tiny workload
    equal the oracle's exact scores on every key of their prefix."""
    print("case: tiny prefill score rows (dense and proxy rows)", flush=True)
    d = to_device(tiny)
    v = oracle.View.of(tiny)
    S = pv.score_rows(d["q"], d["w"], d["k"]).cpu().numpy()
    for t in (0, 1, 63, 64, 1000, 2047):
        assert np.array_equal(S[t][:t + 1].astype(np.float64), oracle.score_row(v, t, t + 1)), t
        assert np.all(np.isnan(S[t][t + 1:])), t
    qbar, _, wbar = pv.proxy_mean(d["q"], d["w"], 4)
    P = pv.score_rows(qbar, wbar, d["k"], pos_mul=4, pos_add=3).cpu().numpy()
    for j in (0, 1, 100, 511):
        pq, _, pw = oracle.proxy(v, 4 * j, 4)
        e = 4 * j + 3
        ref = oracle.score_row(oracle.View("bf16", pq[None], None, pw[None], tiny.k, None), 0, e + 1)
        assert np.array_equal(P[j][:e + 1].astype(np.float64), ref), j
        assert np.all(np.isnan(P[j][e + 1:])), j
    # a window of rows: only rows [row_begin, row_end) are written
    part = pv.score_rows(d["q"], d["w"], d["k"], row_begin=500, row_end=520).cpu().numpy()
    assert np.array_equal(np.nan_to_num(part, nan=-1.0), np.nan_to_num(S[500:520], nan=-1.0))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_decode_scores_exact(dtype):
    """Decode on integer-valued inputs (bf16, and fp8 with unit scales): the
    scores of every mode are exact, except the fp8 proxy's (Reuse), whose fresh
    scale amax/448 is a general binary32 value."""
    print(f"case: decode scores on integer inputs, B=5, {dtype}", flush=True)
    lens = [2, 37, 1000, 999, 1500]
    dec = _decode_inputs(5, lens, g=2, H=8, D=64, Lmax=1500, dtype=dtype)
    d = to_device(dec)
    for mode in ("dense", "reuse", "refine"):
        out, sc = pv.indexer_decode(d["q"], d["w"], d["k"], d["cache_len"], topk=40, C=100, mode=mode,
                                    q_scale=d["q_scale"], k_scale=d["k_scale"], return_scores=True)
        out, sc = out.cpu().numpy(), sc.cpu().numpy()
        for b in range(dec.B):
            v = oracle.decode_view(dec, b)
            ref_rows, _, psc = oracle.decode_seq(dec, b, 40, 100, mode)
            assert np.array_equal(out[b], ref_rows), (mode, b)
            for i in range(2):
                sel = out[b, i][out[b, i] >= 0]
                ref = psc[sel] if mode == "reuse" else oracle.score_list(v, i, sel)
                got = sc[b, i][:len(sel)].astype(np.float64)
                if dtype == "fp8" and mode == "reuse":
                    # the re-quantised proxy carries a general binary32 scale: the
                    # code sum is exact, its two scale products round once each
                    assert np.all(np.abs(got - ref) <= 2.0 ** -22 * np.abs(ref)), (mode, b, i)
                else:
                    assert np.array_equal(got, ref), (mode, b, i)
                assert np.all(np.isnan(sc[b, i][len(sel):]))


@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
def test_float_proxy_bits(dtype):
    # a short sequence (every group checked) and a longer one (sampled groups)
    for L, gs, every in ((203, (8, 2, 1), 1), (2100, (8, 2), 29)):
        print(f"case: {dtype} proxy bits (float inputs, partial last group) L={L}", flush=True)
        inp = synth.dsa_prefill(L=L, H=64, D=128, dtype=dtype, seed=77)
        d = to_device(inp)
        v = oracle.View.of(inp)
        for g in gs:
            qbar, qs, wbar = pv.proxy_mean(d["q"], d["w"], g, q_scale=d.get("q_scale"))
            qbar = qbar.view(torch.int16) if dtype == "bf16" else qbar.view(torch.uint8)
            qbar, qs, wbar = qbar.cpu().numpy(), qs.cpu().numpy(), wbar.cpu().numpy()
            if dtype == "bf16":
                qbar = qbar.view(np.uint16)
            G = (L + g - 1) // g
            for j in sorted(set(range(0, G, every)) | {G - 1}):
                n = min(g, L - j * g)
                c, s, wb = oracle.proxy(v, j * g, n)
                assert np.array_equal(qbar[j], c), (g, j)
                assert qs[j] == s and np.array_equal(wbar[j], wb), (g, j)


SHAPES = [  # (L, H, D, g, topk, C, dtype)
    (1, 4, 32, 4, 8, 16, "bf16"),        # a single query
    (50, 4, 32, 8, 64, 64, "bf16"),       # every row shorter than topk
    (1003, 64, 128, 8, 96, 200, "bf16"),  # partial last group, ragged tiles
    (2049, 33, 64, 16, 128, 256, "bf16"), # ragged key chunk, odd head count
    (10, 2, 32, 16, 3, 5, "bf16"),        # g larger than L
    (700, 1, 256, 5, 40, 80, "bf16"),     # one head, widest D, odd g
    (777, 64, 128, 1, 50, 50, "bf16"),    # g = 1
    (640, 48, 64, 4, 32, 32, "fp8"),      # fp8 codes, C = topk
    (901, 64, 128, 1, 64, 96, "fp8"),
    (300, 7, 256, 3, 17, 40, "fp8"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "L{}H{}D{}g{}k{}C{}{}".format(*s))
def test_shapes_exact(shape):
    L, H, D, g, topk, C_, dt = shape
    print(f"case: exact shape {shape}", flush=True)
    inp = synth.small_integer(L, H, D, seed=L + H + D, qmax=2, kmax=2, wmax=3, dtype=dt)
    modes = ["dense", "reuse", "refine"]
    if dt == "fp8":
        # binary32 sums of fp8 integer codes are exact only without the proxy
        # re-quantisation, i.e. for the dense indexer and one-member groups
        modes = ["dense"] + (["reuse", "refine"] if g == 1 else [])
    for mode in modes:
        got = _run(inp, mode, g, topk, C_)
        ref = _oracle_all(inp, mode, g, topk, C_)
        assert np.array_equal(got, ref), mode


def test_identities_on_gpu():
    print("case: GPU identities (Refine g=1 / C>=L == dense, C=k Refine == Reuse)", flush=True)
    inp = synth.small_integer(1500, 64, 128, seed=9, qmax=2, kmax=2, wmax=3)
    dense = _run(inp, "dense", 1, 100, 100)
    assert np.array_equal(_run(inp, "refine", 1, 100, 100), dense)
    assert np.array_equal(_run(inp, "refine", 8, 100, 1500), dense)
    assert np.array_equal(_run(inp, "reuse", 1, 100, 100), dense)
    assert np.array_equal(_run(inp, "refine", 8, 100, 100), _run(inp, "reuse", 8, 100, 100))


def test_chunked_passes_match_single_pass():
    print("case: minimum workspace (many passes) vs default", flush=True)
    inp = synth.small_integer(3000, 64, 128, seed=4, qmax=2, kmax=2, wmax=3)
    d = to_device(inp)
    for mode in ("dense", "reuse", "refine"):
        big = _run(inp, mode, 8, 128, 256)
        nmin = pv.load().pivot_workspace_min_size(3000, 64, 128, 8, 128, 256, pv._mode(mode), 0)
        ws = torch.empty(nmin, dtype=torch.uint8, device="cuda")
        small = pv.indexer(d["q"], d["w"], d["k"], g=8, topk=128, C=256, mode=mode,
                           workspace=ws).cpu().numpy()
        assert np.array_equal(big, small), mode


def test_long_exact_sampled_groups():
    # L = 32768, H = 64, D = 128 on small integers: the scan runs several key
    # chunks per workgroup row block (longer than the shortest chunk), so chunk
    # edges are checked bit-exactly; whole groups are sampled across the range
    print("case: L=32768 H=64 D=128 integer inputs, Refine g=8, sampled groups", flush=True)
    L, g, topk, C = 32768, 8, 256, 512
    inp = synth.small_integer(L, 64, 128, seed=31, qmax=2, kmax=2, wmax=3)
    out = _run(inp, "refine", g, topk, C)
    v = oracle.View.of(inp)
    G = L // g
    rng = np.random.default_rng(5)
    groups = sorted(set([0, 1, G // 2, G - 2, G - 1]) | set(rng.integers(0, G, 10).tolist()))
    for j in groups:
        ref, _, _ = oracle.group(v, j * g, j * g, g, topk, C, "refine")
        assert np.array_equal(out[j * g:(j + 1) * g], ref), j


@pytest.fixture(scope="module")
def tiny16k():
    return synth.tiny_integer(L=16384, H=4, D=32, seed=77)


@pytest.mark.parametrize("g,W,wmode", [(8, 0, "shared"), (16, 0, "shared"), (8, 300, "excluded"),
                                       (8, 100, "shared")])
def test_refine_2048_groups_bit_exact(tiny16k, g, W, wmode):
    """Refine at 2048 (group, member block) units, the launch shape in which
    every Refine workgroup takes all of its group's candidates, with the
    member top-k on rows of C=256 candidates (one wave per row).  Integer
    inputs: every row, and every returned score, equals the oracle's.  The
    excluded window of 300 leaves the first groups without candidates, so
    their members' rows hold only -1 (and the window)."""
    print(f"case: L=16384 H=4 D=32 Refine g={g} k=64 C=256, window {W} {wmode}", flush=True)
    L, topk, C = 16384, 64, 256
    inp = tiny16k
    d = to_device(inp)
    kw = dict(window=W, window_mode=wmode) if W else dict(return_scores=True)
    res = pv.indexer(d["q"], d["w"], d["k"], g=g, topk=topk, C=C, mode="refine", **kw)
    torch.cuda.synchronize()
    v = oracle.View.of(inp)
    G = L // g
    chunks = np.array_split(np.arange(G), parity.THREADS)
    excl = W if wmode == "excluded" else 0
    parts = parity.pmap(lambda c: oracle.prefill_groups(v, L, g, topk, C, "refine", c, excl=excl)[0], chunks)
    ref = np.concatenate(parts)
    if W:
        ref = oracle.window_union(ref, np.arange(L), W)
        got = res.cpu().numpy()
    else:
        got, sc = res[0].cpu().numpy(), res[1].cpu().numpy()
    bad = np.nonzero((got != ref).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} rows differ, first {bad[:5]}"
    if W:
        return
    def row_scores(rows):
        for t in rows:
            sel = got[t][got[t] >= 0]
            assert np.array_equal(sc[t][:len(sel)].astype(np.float64), oracle.score_list(v, int(t), sel)), t
            assert np.all(np.isnan(sc[t][len(sel):])), t
    parity.pmap(row_scores, np.array_split(np.arange(L), parity.THREADS))


@pytest.mark.parametrize("kmax", [4, 0])
def test_long_rows_selection(kmax):
    # rows of 30720 scores or more are sampled before their first pass; with
    # spread-out integer scores the sampled estimate lets one pass gather the
    # candidates, with all-zero keys (every score equal) it cannot and the
    # selection falls back to passes over the row: both must be exact
    print(f"case: L=40000 H=8 D=64 integer inputs, kmax={kmax}, long-row top-k", flush=True)
    L, g, topk, C = 40000, 8, 2048, 4096
    inp = synth.small_integer(L, 8, 64, seed=41, qmax=4, kmax=kmax, wmax=3)
    v = oracle.View.of(inp)
    G = L // g
    rng = np.random.default_rng(9)
    out = _run(inp, "refine", g, topk, C)
    cand = pv.candidates(*(to_device(inp)[x] for x in ("q", "w", "k")), g=g, topk=topk, C=C,
                         mode="refine").cpu().numpy()
    groups = sorted({0, 3839, 3840, G - 2, G - 1} | set(rng.integers(3840, G, 6).tolist()))
    for j in groups:
        ref, rc, _ = oracle.group(v, j * g, j * g, g, topk, C, "refine")
        assert np.array_equal(cand[j], rc), j
        assert np.array_equal(out[j * g:(j + 1) * g], ref), j
    dense = _run(inp, "dense", 1, topk, topk)
    rows = np.array(sorted({30719, 30720, L - 1} | set(rng.integers(30720, L, 5).tolist())))
    assert np.array_equal(dense[rows], oracle.dense_rows(v, rows, topk))


@pytest.mark.parametrize("kmax", [4, 0])
def test_long_rows_few_rows_selection(kmax):
    # fewer than 512 proxy rows in a launch take the 1024-thread long-row
    # top-k (many rows take the 512-thread one above): g = 128 at L = 40000
    # gives 313 proxy rows, the last 74 of them 30720 scores or longer
    print(f"case: L=40000 H=8 D=64 integer inputs, g=128, kmax={kmax}, few long rows", flush=True)
    L, g, topk, C = 40000, 128, 2048, 4096
    inp = synth.small_integer(L, 8, 64, seed=43, qmax=4, kmax=kmax, wmax=3)
    v = oracle.View.of(inp)
    G = (L + g - 1) // g
    cand = pv.candidates(*(to_device(inp)[x] for x in ("q", "w", "k")), g=g, topk=topk, C=C,
                         mode="refine").cpu().numpy()
    rng = np.random.default_rng(10)
    for j in sorted({0, 238, 239, G - 2, G - 1} | set(rng.integers(240, G, 4).tolist())):
        _, rc, _ = oracle.group(v, j * g, j * g, min(g, L - j * g), topk, C, "refine")
        assert np.array_equal(cand[j], rc), j


def test_deterministic_repeat():
    # float inputs (where a different summation order would show), ten calls
    # each: a prefill whose long rows take the sampled top-k, and a decode step
    print("case: repeated calls are identical (prefill L=40000, decode B=8)", flush=True)
    inp = synth.dsa_prefill(L=40000, H=64, D=128, seed=12)
    d = to_device(inp)
    ws = torch.empty(pv.workspace_size(40000, 64, 128, 8, 256, 512, "refine", 0), dtype=torch.uint8,
                     device="cuda")
    runs = [pv.indexer(d["q"], d["w"], d["k"], g=8, topk=256, C=512, mode="refine",
                       workspace=ws).cpu().numpy() for _ in range(10)]
    assert all(np.array_equal(runs[0], r) for r in runs[1:])
    dec = synth.decode_mtp(B=8, Lmin=4000, Lmax=40000, H=64, D=128, g=2, seed=77)
    dd = to_device(dec)
    outs = [pv.indexer_decode(dd["q"], dd["w"], dd["k"], dd["cache_len"], topk=256, C=512,
                              mode="refine", q_scale=dd["q_scale"], k_scale=dd["k_scale"]).cpu().numpy()
            for _ in range(10)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


def _decode_inputs(B, lens, g, H=8, D=64, dtype="bf16", Lmax=None, seed=3):
    Lmax = Lmax or max(lens)
    rng = np.random.default_rng(seed)
    qf = rng.integers(-2, 3, (B, g, H, D)).astype(np.float32)
    kf = rng.integers(-2, 3, (B, Lmax, D)).astype(np.float32)
    w = rng.integers(1, 4, (B, g, H)).astype(np.float32)
    if dtype == "bf16":
        return synth.DecodeInputs("bf16", B, Lmax, H, D, g, synth.encode_bf16(qf), None, w,
                                  synth.encode_bf16(kf), None, np.asarray(lens, np.int32))
    return synth.DecodeInputs("fp8", B, Lmax, H, D, g, synth._encode_fp8(qf),
                              np.ones((B, g), np.float32), w, synth._encode_fp8(kf),
                              np.ones((B, Lmax), np.float32), np.asarray(lens, np.int32))


@pytest.mark.parametrize("mode", ["dense", "reuse", "refine"])
def test_decode_exact(mode):
    print(f"case: decode exact B=5 g=2 {mode}", flush=True)
    lens = [2, 37, 1000, 999, 1500]
    dec = _decode_inputs(5, lens, g=2, H=8, D=64, Lmax=1500)
    d = to_device(dec)
    out = pv.indexer_decode(d["q"], d["w"], d["k"], d["cache_len"], topk=40, C=100,
                            mode=mode).cpu().numpy()
    for b in range(5):
        ref, _, _ = oracle.decode_seq(dec, b, 40, 100, mode)
        assert np.array_equal(out[b], ref), b


@pytest.mark.parametrize("dtype,mode", [("bf16", "dense"), ("bf16", "refine"), ("fp8", "refine")])
def test_decode_exact_many_sequences(dtype, mode):
    # about 1100 key pairs over the batch: the decode scan's per-workgroup
    # runs of pairs start and end inside sequences and span several of them
    print(f"case: decode exact B=24 H=64 D=128 {dtype} {mode}", flush=True)
    rng = np.random.default_rng(21)
    lens = [int(x) for x in rng.integers(2, 6000, 24)]
    lens[3], lens[7], lens[8], lens[9] = 6000, 64, 65, 2
    dec = _decode_inputs(24, lens, g=2, H=64, D=128, dtype=dtype, Lmax=6000, seed=22)
    d = to_device(dec)
    kw = dict(q_scale=d["q_scale"], k_scale=d["k_scale"]) if dtype == "fp8" else {}
    out = pv.indexer_decode(d["q"], d["w"], d["k"], d["cache_len"], topk=64, C=256, mode=mode,
                            **kw).cpu().numpy()
    for b in range(24):
        ref, _, _ = oracle.decode_seq(dec, b, 64, 256, mode)
        assert np.array_equal(out[b], ref), b


@pytest.mark.parametrize("mode", ["dense", "refine"])
def test_decode_exact_many_short_sequences(mode):
    # B = 300 > 256: the decode scan's division of the batch into per-workgroup
    # runs counts sequences in several blocks; short and invalid lengths mixed
    print(f"case: decode exact B=300 H=8 D=64 bf16 {mode}", flush=True)
    rng = np.random.default_rng(41)
    lens = [int(x) for x in rng.integers(2, 700, 300)]
    lens[0], lens[17], lens[255], lens[256], lens[299] = 1, 0, 700, 64, 2
    dec = _decode_inputs(300, lens, g=2, H=8, D=64, Lmax=700, seed=42)
    d = to_device(dec)
    out = pv.indexer_decode(d["q"], d["w"], d["k"], d["cache_len"], topk=32, C=96,
                            mode=mode).cpu().numpy()
    for b in range(300):
        if lens[b] < 2:
            assert np.all(out[b] == -1), b
            continue
        ref, _, _ = oracle.decode_seq(dec, b, 32, 96, mode)
        assert np.array_equal(out[b], ref), b


@pytest.mark.parametrize("dtype,D", [("fp8", 64), ("fp8", 256), ("bf16", 32), ("bf16", 256)])
@pytest.mark.parametrize("mode", ["dense", "refine"])
def test_decode_exact_head_dims(dtype, D, mode):
    # every key width has its own decode-scan geometry (waves per workgroup,
    # ring depth); sequences end inside and across the workgroups' runs
    print(f"case: decode exact B=12 H=16 D={D} {dtype} {mode}", flush=True)
    rng = np.random.default_rng(D + (dtype == "fp8"))
    lens = [int(x) for x in rng.integers(2, 3000, 12)]
    lens[1], lens[5], lens[6] = 3000, 64, 2
    dec = _decode_inputs(12, lens, g=2, H=16, D=D, dtype=dtype, Lmax=3000, seed=D)
    d = to_device(dec)
    kw = dict(q_scale=d["q_scale"], k_scale=d["k_scale"]) if dtype == "fp8" else {}
    out = pv.indexer_decode(d["q"], d["w"], d["k"], d["cache_len"], topk=48, C=160, mode=mode,
                            **kw).cpu().numpy()
    for b in range(12):
        ref, _, _ = oracle.decode_seq(dec, b, 48, 160, mode)
        assert np.array_equal(out[b], ref), b


def test_decode_matches_last_prefill_group_and_rejects_bad_lengths():
    print("case: decode == last prefill group; invalid cache lengths give -1 rows", flush=True)
    g = 4
    inp = synth.small_integer(400, 16, 64, seed=8, qmax=2, kmax=2, wmax=3)
    pre = _run(inp, "refine", g, 30, 60)
    dec = synth.DecodeInputs("bf16", 1, 400, 16, 64, g, inp.q[None, -g:], None,
                             inp.w[None, -g:], inp.k[None], None, np.array([400], np.int32))
    d = to_device(dec)
    out = pv.indexer_decode(d["q"], d["w"], d["k"], d["cache_len"], topk=30, C=60,
                            mode="refine").cpu().numpy()
    assert np.array_equal(out[0], pre[-g:])
    bad = _decode_inputs(3, [1, 0, 70], g=2, H=4, D=32, Lmax=64)
    d = to_device(bad)
    d["cache_len"] = torch.tensor([1, 0, 70], dtype=torch.int32, device="cuda")
    for mode in ("dense", "reuse", "refine"):
        out = pv.indexer_decode(d["q"], d["w"], d["k"], d["cache_len"], topk=8, C=16,
                                mode=mode).cpu().numpy()
        assert np.all(out == -1), mode


def test_decode_fp8_exact_dense():
    print("case: decode fp8 integer codes, dense", flush=True)
    dec = _decode_inputs(4, [64, 500, 2000, 3], g=3, H=64, D=128, dtype="fp8", Lmax=2000)
    d = to_device(dec)
    out = pv.indexer_decode(d["q"], d["w"], d["k"], d["cache_len"], topk=50, C=50, mode="dense",
                            q_scale=d["q_scale"], k_scale=d["k_scale"]).cpu().numpy()
    for b in range(4):
        ref, _, _ = oracle.decode_seq(dec, b, 50, 50, "dense")
        assert np.array_equal(out[b], ref), b


@pytest.mark.parametrize("g", [3, 4, 8])
@pytest.mark.parametrize("mode", ["dense", "reuse", "refine"])
def test_decode_deeper_mtp_groups(g, mode):
    # more than two tokens per multi-token-prediction step: the group is the g
    # queries decoded together, the proxy their mean over the whole cache
    print(f"case: decode MTP group g={g} B=10 H=16 D=64 bf16 {mode}", flush=True)
    rng = np.random.default_rng(g)
    lens = [int(x) for x in rng.integers(g, 2500, 10)]
    lens[2], lens[6] = g, g - 1  # the smallest valid cache and an invalid one
    dec = _decode_inputs(10, lens, g=g, H=16, D=64, Lmax=2500, seed=60 + g)
    d = to_device(dec)
    out = pv.indexer_decode(d["q"], d["w"], d["k"], d["cache_len"], topk=40, C=120,
                            mode=mode).cpu().numpy()
    assert out.shape == (10, g, 40)
    for b in range(10):
        if lens[b] < g:
            assert np.all(out[b] == -1), b
            continue
        ref, _, _ = oracle.decode_seq(dec, b, 40, 120, mode)
        assert np.array_equal(out[b], ref), b
