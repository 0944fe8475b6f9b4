"""Pins of the CPU oracle against facts that do not come from the oracle itself:
the pages' printed worked example, a hand-derived PIVOT example, library
routines (PyTorch's fp8/bf16 casts, numpy dot), brute-force enumeration, exact
rational arithmetic and closed forms.  CPU only."""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import GOLDEN


def _bf16_view(q, w, k):
    q = np.asarray(q, np.float32)
    k = np.asarray(k, np.float32)
    return oracle.View("bf16", synth.encode_bf16(q), None, np.asarray(w, np.float32),
                       synth.encode_bf16(k), None)


# ----------------------------------------------------------------------------
# number formats, pinned to PyTorch's casts
# ----------------------------------------------------------------------------

def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(c) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ref[~nan], got[~nan])
    assert oracle.e4m3_value(0x7E) == 448.0 and oracle.e4m3_value(0x01) == 2.0 ** -9


def _torch_e4m3(x):
    x = np.clip(np.asarray(x, np.float32), -448, 448)
    return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_every_value_midpoint_and_overflow():
    vals = np.array([oracle.e4m3_value(c) for c in range(0x7F)], np.float64)
    mids = (vals[:-1] + vals[1:]) / 2  # exact ties: must go to the even code
    probes = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                             [448.0, 449.0, 464.0, 465.0, 1e6, 3.4e38, 1e-30, 0.0]])
    probes = probes.astype(np.float32)
    probes = np.concatenate([probes, -probes])
    rng = np.random.default_rng(7)
    rnd = (rng.standard_normal(20000) * np.exp(rng.uniform(-12, 7, 20000))).astype(np.float32)
    allx = np.concatenate([probes, rnd])
    got = np.array([oracle.e4m3_from_f32(x) for x in allx], np.uint8)
    ref = _torch_e4m3(allx)
    # torch keeps the sign of an underflow to zero; so does the oracle
    assert np.array_equal(got, ref)
    # ties go to the even code
    for i, m in enumerate(mids.astype(np.float32)):
        c = oracle.e4m3_from_f32(m)
        assert c % 2 == 0 and c in (i, i + 1)
    assert oracle.e4m3_from_f32(1e9) == 0x7E and oracle.e4m3_from_f32(-1e9) == 0xFE


def test_bf16_codec_matches_torch():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(50000) * np.exp(rng.uniform(-60, 60, 50000))).astype(np.float32)
    # exact ties: a bf16 value plus half of its last place
    base = synth.encode_bf16(rng.standard_normal(2000).astype(np.float32))
    ties = ((base.astype(np.uint32) << 16) | 0x8000).view(np.float32)
    allx = np.concatenate([x, ties, np.float32([0.0, -0.0, 3.3895314e38, 1e-40, -1e-40])])
    got = np.array([oracle.bf16_from_f32(v) for v in allx], np.uint16)
    ref = torch.from_numpy(allx).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    codes = rng.integers(0, 1 << 16, 5000).astype(np.uint16)
    dec = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    mine = np.array([oracle.bf16_value(c) for c in codes])
    fin = np.isfinite(dec)
    assert np.array_equal(dec[fin], mine[fin])
    assert np.array_equal(np.isnan(dec), np.isnan(mine))


# ----------------------------------------------------------------------------
# the pages' printed worked example
# ----------------------------------------------------------------------------

def _fig1_view():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_fig1.json")))
    a = ex["keys_first_component"]
    b = ex["keys_second_component_p0_to_p6"] + [ex["key_p7_second_component"]]
    k = np.stack([a, b], axis=1)
    q = np.zeros((8, 1, 2), np.float32)
    q[6, 0] = ex["query_p6"]
    q[7, 0] = ex["query_p7"]
    q[:6, 0] = [1.0, 0.0]
    return ex, _bf16_view(q, np.ones((8, 1)), k)


def test_worked_example_scores_and_top3():
    ex, v = _fig1_view()
    s7 = oracle.score_row(v, 7, 8)
    s6 = oracle.score_row(v, 6, 7)
    # printed decimals are stored as bf16: agree to bf16 precision
    assert np.allclose(s7, ex["scores_p7"], rtol=2 ** -8, atol=0)
    assert np.allclose(s6, ex["scores_p6"], rtol=2 ** -8, atol=0)
    out = oracle.dense_rows(v, [7, 6], ex["topk"])
    assert out[0].tolist() == ex["top3_p7"]
    assert out[1].tolist() == ex["top3_p6"]  # 7 excluded although its score is largest


def test_worked_example_as_one_decode_group():
    # the same positions as a decode MTP group of g=2 (queries p6, p7), dense mode
    ex, v = _fig1_view()
    out, _, _ = oracle.group(v, 6, 6, 2, 3, 3, "dense")
    assert out.tolist() == [ex["top3_p6"], ex["top3_p7"]]


# ----------------------------------------------------------------------------
# sliding window added to the selection (printed Figure 3 union; the
# excluded-window design derived by hand from the printed Figure 1 scores)
# ----------------------------------------------------------------------------

def _window_example():
    return json.load(open(os.path.join(GOLDEN, "window_example_fig3.json")))


def test_window_union_printed_example():
    ex, v = _fig1_view()
    wx = _window_example()
    W = wx["window"]
    sel = oracle.dense_rows(v, [7, 6], ex["topk"])
    out = oracle.window_union(sel, [7, 6], W)
    assert out.shape == (2, ex["topk"] + W)
    got7 = [int(p) for p in out[0] if p >= 0]
    assert got7 == wx["union_p7_printed"]
    assert len(got7) == wx["positions_read_p7_printed"]  # 7 is read once
    assert set(wx["window_p7"]) <= set(got7)
    assert out[0].tolist()[len(got7):] == [-1] * (ex["topk"] + W - len(got7))
    assert [int(p) for p in out[1] if p >= 0] == wx["union_p6_derived"]
    # window 0 leaves a selection unchanged; window 1 adds the query's own position
    assert oracle.window_union(sel, [7, 6], 0).tolist() == sel.tolist()
    assert [int(p) for p in oracle.window_union(sel, [7, 6], 1)[1] if p >= 0] == [1, 3, 6]


def test_window_excluded_derived_example():
    ex, v = _fig1_view()
    wx = _window_example()
    W = wx["window"]
    sel = oracle.dense_rows(v, [7, 6], ex["topk"], excl=W)
    out = oracle.window_union(sel, [7, 6], W)
    assert out[0].tolist() == wx["excluded_p7_derived"]  # all k + W slots used
    assert out[1].tolist() == wx["excluded_p6_derived"]
    # as one decode group (p6, p7): the same rows
    rows, _, _ = oracle.group(v, 6, 6, 2, ex["topk"], ex["topk"], "dense", excl=W)
    assert rows.tolist() == sel[::-1].tolist()
    # a window as long as the prefix leaves nothing to choose
    assert oracle.dense_rows(v, [2], 3, excl=3).tolist() == [[-1, -1, -1]]
    assert oracle.window_union(oracle.dense_rows(v, [2], 3, excl=3), [2], 3).tolist() == \
        [[0, 1, 2, -1, -1, -1]]


# ----------------------------------------------------------------------------
# hand-derived PIVOT example (integers, exact)
# ----------------------------------------------------------------------------

def _derived():
    ex = json.load(open(os.path.join(GOLDEN, "derived_pivot_example.json")))
    k = np.stack([ex["a"], ex["b"]], axis=1)
    q = np.zeros((8, 1, 2), np.float32)
    q[:6, 0] = [[1, 0], [0, 1]] * 3
    q[6, 0] = ex["q6"]
    q[7, 0] = ex["q7"]
    return ex, _bf16_view(q, np.ones((8, 1)), k)


def test_derived_pivot_example_reuse_refine():
    ex, v = _derived()
    codes, s, wbar = oracle.proxy(v, 6, 2)
    assert [oracle.bf16_value(c) for c in codes[0]] == ex["proxy"] and s == 1.0 and wbar[0] == 1
    out, ptop, psc = oracle.group(v, 6, 6, 2, 3, 4, "reuse")
    assert psc.tolist() == ex["proxy_scores"]
    assert ptop.tolist() == ex["reuse_k3"]["ptop"]
    assert out.tolist() == [ex["reuse_k3"]["member6"], ex["reuse_k3"]["member7"]]
    out, cand, _ = oracle.group(v, 6, 6, 2, 3, 4, "refine")
    assert cand.tolist() == ex["refine_k3_C4"]["cand"]
    assert out.tolist() == [ex["refine_k3_C4"]["member6"], ex["refine_k3_C4"]["member7"]]
    out, _, _ = oracle.group(v, 6, 6, 2, 3, 8, "refine")
    assert out.tolist() == [ex["refine_k3_C8"]["member6"], ex["refine_k3_C8"]["member7"]]
    # the prefill grouping (L=8, g=2) reaches the same rows through group 3
    rows, cand = oracle.prefill_groups(v, 8, 2, 3, 4, "refine", [3])
    assert rows.tolist() == [ex["refine_k3_C4"]["member6"], ex["refine_k3_C4"]["member7"]]


# ----------------------------------------------------------------------------
# score: special cases that reduce to library routines / exact rationals
# ----------------------------------------------------------------------------

def test_score_single_head_is_plain_dot_product():
    rng = np.random.default_rng(3)
    D = 16
    q = rng.integers(1, 4, (1, 1, D)).astype(np.float32)  # positive: ReLU inactive
    k = rng.integers(1, 4, (5, D)).astype(np.float32)
    v = _bf16_view(q, np.ones((1, 1)), k)
    assert oracle.score_row(v, 0, 5).tolist() == (k @ q[0, 0]).astype(np.float64).tolist()


def test_score_relu_drops_negative_heads_and_weights_scale_linearly():
    # head 0 has a negative dot product with the key, head 1 a positive one
    q = np.array([[[-1, -2], [3, 1]]], np.float32)
    k = np.array([[2, 1]], np.float32)
    v = _bf16_view(q, [[5.0, 0.5]], k)
    assert oracle.score_row(v, 0, 1)[0] == 0.5 * 7
    v2 = _bf16_view(q, [[5.0, 1.0]], k)
    assert oracle.score_row(v2, 0, 1)[0] == 7.0
    # all heads negative -> score exactly zero
    v3 = _bf16_view(-np.abs(q), [[5.0, 1.0]], k)
    assert oracle.score_row(v3, 0, 1)[0] == 0.0


def test_score_exact_on_integer_inputs():
    inp = synth.small_integer(L=12, H=3, D=5, seed=5)
    v = oracle.View.of(inp)
    qf = inp.q.astype(np.uint32) << 16
    qv = qf.view(np.float32).astype(np.int64)
    kv = (inp.k.astype(np.uint32) << 16).view(np.float32).astype(np.int64)
    for t in range(12):
        got = oracle.score_row(v, t, 12)
        for s in range(12):
            exact = sum(Fraction(float(inp.w[t, h])) * max(0, int(qv[t, h] @ kv[s]))
                        for h in range(3))
            assert Fraction(got[s]) == exact


def test_fp8_score_is_scaled_code_score():
    inp = synth.small_integer(L=6, H=2, D=4, seed=9, dtype="fp8")
    inp.q_scale = np.float32([0.5, 2.0, 0.25, 1.0, 4.0, 0.125])
    inp.k_scale = np.float32([2.0, 0.5, 1.0, 8.0, 0.25, 1.0])
    v = oracle.View.of(inp)
    v1 = oracle.View("fp8", inp.q, np.ones(6, np.float32), inp.w, inp.k, np.ones(6, np.float32))
    for t in range(6):
        a = oracle.score_row(v, t, 6)
        b = oracle.score_row(v1, t, 6)
        assert np.array_equal(a, b * inp.q_scale[t] * inp.k_scale[:6].astype(np.float64))


# ----------------------------------------------------------------------------
# top-m: brute-force enumeration on tiny inputs
# ----------------------------------------------------------------------------

def _brute_topk(scores, pos, m):
    """Every subset of size min(m, n); keep those in which each chosen element
    beats each unchosen one (higher score, or equal score and lower position).
    The rule is a strict total order, so exactly one subset survives."""
    n = len(pos)
    r = min(m, n)
    winners = []
    for sub in itertools.combinations(range(n), r):
        chosen = set(sub)
        ok = all(
            (scores[i] > scores[j]) or (scores[i] == scores[j] and pos[i] < pos[j])
            for i in chosen for j in range(n) if j not in chosen)
        if ok:
            winners.append(sorted(pos[i] for i in sub))
    assert len(winners) == 1
    return winners[0] + [-1] * (m - r)


@pytest.mark.parametrize("seed", range(12))
def test_topk_bruteforce(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 9))
    scores = rng.integers(0, 4, n).astype(np.float64)  # many ties
    if seed % 3 == 0 and n:
        scores[0] = -0.0
        scores[-1] = 0.0
    pos = np.sort(rng.choice(40, n, replace=False)).astype(np.int32)
    for m in range(1, 7):
        assert oracle.topk(scores, m, pos).tolist() == _brute_topk(list(scores), list(pos), m)


@pytest.mark.parametrize("seed", range(6))
def test_dense_and_refine_bruteforce_tiny(seed):
    """Dense rows and Refine rows equal the brute-force selection over their pools."""
    rng = np.random.default_rng(100 + seed)
    L = int(rng.integers(3, 10))
    H = int(rng.integers(1, 3))
    D = int(rng.integers(1, 4))
    inp = synth.small_integer(L, H, D, seed=200 + seed, qmax=2, kmax=2, wmax=2)
    v = oracle.View.of(inp)
    k = int(rng.integers(1, 5))
    dense = oracle.dense_rows(v, np.arange(L), k)
    for t in range(L):
        sc = oracle.score_row(v, t, t + 1)
        assert dense[t].tolist() == _brute_topk(list(sc), list(range(t + 1)), k)
    for g in range(1, L + 1):
        C_ = k + int(rng.integers(0, 3))
        G = (L + g - 1) // g
        rows, cand = oracle.prefill_groups(v, L, g, k, C_, "refine", np.arange(G))
        r = 0
        for j in range(G):
            members = range(j * g, min(L, j * g + g))
            e = members[-1]
            # candidates: the proxy's own top-C over [0, e]
            pq, ps, pw = oracle.proxy(v, j * g, len(members))
            pv = oracle.View("bf16", pq[None], None, pw[None], inp.k, None)
            psc = oracle.score_row(pv, 0, e + 1)
            assert cand[j].tolist() == _brute_topk(list(psc), list(range(e + 1)), C_)
            for t in members:
                pool = [c for c in cand[j] if 0 <= c <= t]
                sc = oracle.score_pairs(v, [t] * len(pool), pool) if pool else []
                assert rows[r].tolist() == _brute_topk(list(sc), pool, k)
                r += 1


# ----------------------------------------------------------------------------
# proxy mean: closed forms
# ----------------------------------------------------------------------------

def test_proxy_mean_exact_rational_on_integer_inputs():
    inp = synth.tiny_integer(L=64, H=4, D=32, seed=1)
    v = oracle.View.of(inp)
    qv = (inp.q.astype(np.uint32) << 16).view(np.float32)
    for g in (2, 3, 4, 8, 16):
        for j in range(0, (64 + g - 1) // g):
            n = min(g, 64 - j * g)
            codes, s, wbar = oracle.proxy(v, j * g, n)
            mean = qv[j * g:j * g + n].astype(np.float64).mean(axis=0)
            got = (codes.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            if n in (1, 2, 4, 8, 16):  # multiples of 1/(8n): exact in bf16
                assert np.array_equal(got, mean)
            else:  # otherwise the nearest bf16 of the binary32 mean
                assert np.all(np.abs(got - mean) <= np.abs(mean) * 2 ** -8 + 1e-30)
            assert np.allclose(wbar, inp.w[j * g:j * g + n].mean(axis=0), rtol=2 ** -23)
            assert s == 1.0


def test_proxy_fp8_scale_and_codes():
    inp = synth.dsa_prefill(L=32, H=4, D=32, dtype="fp8", seed=3)
    v = oracle.View.of(inp)
    deq = inp.q_scale[:, None, None] * torch.from_numpy(inp.q).view(
        torch.float8_e4m3fn).float().numpy()
    for j in range(4):
        codes, s, wbar = oracle.proxy(v, j * 8, 8)
        mean = np.zeros((4, 32), np.float32)
        for t in range(j * 8, j * 8 + 8):
            mean = mean + deq[t]
        mean = mean / np.float32(8)
        amax = np.abs(mean).max()
        assert s == np.float32(amax / np.float32(448))
        assert np.array_equal(codes, _torch_e4m3(mean / s))
    # a single-member group is the member itself
    codes, s, wbar = oracle.proxy(v, 5, 1)
    assert np.array_equal(codes, inp.q[5]) and s == inp.q_scale[5]


def test_tiny_config_scores_are_exact_multiples():
    """Closed form: q,k in {-4..4}/8, w in {1..4}/8, D=32, H=4 -> every score is a
    multiple of 2^-9 below 2^6, so binary32 and double sums are both exact."""
    inp = synth.tiny_integer(L=256, seed=1001)
    v = oracle.View.of(inp)
    for t in (0, 17, 255):
        s = oracle.score_row(v, t, t + 1)
        assert np.all(s * 2 ** 9 == np.round(s * 2 ** 9))
        assert np.all(np.abs(s) < 2 ** 6)
        assert np.array_equal(s.astype(np.float32).astype(np.float64), s)


@pytest.mark.parametrize("seed", range(6))
def test_window_excluded_bruteforce_tiny(seed):
    """With the window excluded, dense and Refine rows are the brute-force
    selection over positions 0..t-W; the proxy's candidates over 0..e-W."""
    rng = np.random.default_rng(300 + seed)
    L = int(rng.integers(3, 10))
    H = int(rng.integers(1, 3))
    D = int(rng.integers(1, 4))
    inp = synth.small_integer(L, H, D, seed=400 + seed, qmax=2, kmax=2, wmax=2)
    v = oracle.View.of(inp)
    k = int(rng.integers(1, 5))
    W = int(rng.integers(1, 4))
    dense = oracle.dense_rows(v, np.arange(L), k, excl=W)
    for t in range(L):
        n = max(t - W + 1, 0)
        sc = oracle.score_row(v, t, n) if n else []
        assert dense[t].tolist() == _brute_topk(list(sc), list(range(n)), k)
    for g in range(1, L + 1):
        C_ = k + int(rng.integers(0, 3))
        G = (L + g - 1) // g
        rows, cand = oracle.prefill_groups(v, L, g, k, C_, "refine", np.arange(G), excl=W)
        r = 0
        for j in range(G):
            members = range(j * g, min(L, j * g + g))
            ne = max(members[-1] - W + 1, 0)
            pq, ps, pw = oracle.proxy(v, j * g, len(members))
            pv = oracle.View("bf16", pq[None], None, pw[None], inp.k, None)
            psc = oracle.score_row(pv, 0, ne) if ne else []
            assert cand[j].tolist() == _brute_topk(list(psc), list(range(ne)), C_)
            for t in members:
                pool = [c for c in cand[j] if 0 <= c <= t - W]
                sc = oracle.score_pairs(v, [t] * len(pool), pool) if pool else []
                assert rows[r].tolist() == _brute_topk(list(sc), pool, k)
                r += 1
