"""Exact identities the method fixes (arXiv:2607.24593 abstract: Refine re-scores
the proxy's candidate set with each member's own indexer; Reuse shares the proxy
top-k), checked on the oracle with integer-valued inputs where every score is
exact.  CPU only."""
import numpy as np
import pytest

import oracle
import synth

CASES = [  # (L, H, D, topk, seed, dtype)
    (37, 2, 4, 5, 1, "bf16"),
    (64, 3, 8, 9, 2, "bf16"),
    (50, 2, 6, 4, 3, "fp8"),
]


def _all_groups(v, L, g, k, C_, mode):
    G = (L + g - 1) // g
    return oracle.prefill_groups(v, L, g, k, C_, mode, np.arange(G))


@pytest.fixture(params=CASES, ids=lambda c: f"L{c[0]}H{c[1]}D{c[2]}k{c[3]}{c[5]}")
def case(request):
    L, H, D, k, seed, dtype = request.param
    inp = synth.small_integer(L, H, D, seed=seed, dtype=dtype)
    v = oracle.View.of(inp)
    dense = oracle.dense_rows(v, np.arange(L), k)
    return L, k, inp, v, dense


def test_causality_and_valid_counts(case):
    L, k, inp, v, dense = case
    for g in (1, 2, 3, 8):
        for mode in ("reuse", "refine"):
            rows, _ = _all_groups(v, L, g, k, k + g - 1 + 2, mode)
            for t in range(L):
                r = rows[t]
                valid = r[r >= 0]
                assert np.all(valid <= t)                          # I7: no future position
                assert np.all(np.diff(valid) > 0)                  # ascending, distinct
                assert np.all(r[len(valid):] == -1)                # -1 only at the tail
                if mode == "refine":
                    assert len(valid) == min(k, t + 1)             # I9 (C >= k+g-1)
    for t in range(L):
        assert np.sum(dense[t] >= 0) == min(k, t + 1)


def test_refine_g1_equals_dense(case):          # I1
    L, k, inp, v, dense = case
    for C_ in (k, k + 3, L):
        rows, _ = _all_groups(v, L, 1, k, C_, "refine")
        assert np.array_equal(rows, dense)


def test_refine_full_candidates_equals_dense(case):  # I2: C >= e_j + 1 for every g
    L, k, inp, v, dense = case
    for g in (2, 3, 5, 8, L):
        rows, _ = _all_groups(v, L, g, k, L, "refine")
        assert np.array_equal(rows, dense)


def test_reuse_g1_equals_dense(case):           # I3
    L, k, inp, v, dense = case
    rows, _ = _all_groups(v, L, 1, k, k, "reuse")
    assert np.array_equal(rows, dense)


def test_refine_with_C_equal_k_is_reuse(case):  # I4
    L, k, inp, v, dense = case
    for g in (2, 4, 7):
        a, _ = _all_groups(v, L, g, k, k, "refine")
        b, _ = _all_groups(v, L, g, k, k, "reuse")
        assert np.array_equal(a, b)


def test_reuse_last_member_gets_proxy_topk(case):  # I5
    L, k, inp, v, dense = case
    g = 4
    rows, ptop = _all_groups(v, L, g, k, k, "reuse")
    for j in range((L + g - 1) // g):
        last = min(L, j * g + g) - 1
        assert np.array_equal(rows[last], ptop[j])
        for t in range(j * g, last + 1):  # every member gets the prefix of ptop up to t
            exp = [p for p in ptop[j] if 0 <= p <= t]
            assert rows[t].tolist() == exp + [-1] * (k - len(exp))


def test_refine_subset_and_overlap_identity(case):  # I6 and I8
    L, k, inp, v, dense = case
    g, C_ = 4, k + 4
    rows, cand = _all_groups(v, L, g, k, C_, "refine")
    for t in range(L):
        j = t // g
        c = set(cand[j][cand[j] >= 0].tolist())
        r = set(rows[t][rows[t] >= 0].tolist())
        d = set(dense[t][dense[t] >= 0].tolist())
        assert r <= {p for p in c if p <= t}
        assert len(r & d) == len(d & c)


def test_doubling_weights_or_queries_changes_nothing(case):  # I10
    L, k, inp, v, dense = case
    w2 = oracle.View(inp.dtype, inp.q, inp.q_scale, inp.w * 2, inp.k, inp.k_scale)
    if inp.dtype == "bf16":
        q2 = synth.encode_bf16(((inp.q.astype(np.uint32) << 16).view(np.float32)) * 2)
        qv2 = oracle.View("bf16", q2, None, inp.w, inp.k, None)
    else:
        qv2 = oracle.View("fp8", inp.q, inp.q_scale * 2, inp.w, inp.k, inp.k_scale)
    for vv in (w2, qv2):
        assert np.array_equal(oracle.dense_rows(vv, np.arange(L), k), dense)
        for mode in ("reuse", "refine"):
            a, _ = _all_groups(v, L, 4, k, k + 3, mode)
            b, _ = _all_groups(vv, L, 4, k, k + 3, mode)
            assert np.array_equal(a, b)


def test_decode_group_equals_last_prefill_group():  # I11
    for dtype in ("bf16", "fp8"):
        g, k, C_ = 3, 5, 9
        L = 30
        inp = synth.small_integer(L, 2, 4, seed=42, dtype=dtype)
        v = oracle.View.of(inp)
        for mode in ("reuse", "refine", "dense"):
            rows, cand = oracle.prefill_groups(v, L, g, k, C_, mode, [L // g - 1])
            # the same sequence as a decode step: cache of L keys, last g queries
            dv = oracle.View(dtype, inp.q[L - g:], None if inp.q_scale is None
                             else inp.q_scale[L - g:], inp.w[L - g:], inp.k, inp.k_scale)
            out, dc, _ = oracle.group(dv, 0, L - g, g, k, C_, mode)
            assert np.array_equal(out, rows)
            if mode != "dense":
                assert np.array_equal(dc, cand[0])


# ----------------------------------------------------------------------------
# sliding window (tutorial "Sparse Attention의 Indexer", section on combining
# the recent window with the selected positions): the shared window is a union,
# the excluded window moves every query's limit from t to t - W
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("W", [1, 3, 7])
def test_window_excluded_identities(case, W):
    L, k, inp, v, dense = case
    dense_x = oracle.dense_rows(v, np.arange(L), k, excl=W)
    for t in range(L):
        r = dense_x[t][dense_x[t] >= 0]
        assert np.all(r <= t - W) and len(r) == min(k, max(0, t - W + 1))
    for g in (1, 2, 3, 8):
        rows, _ = _all_groups_x(v, L, g, k, L, "refine", W)
        assert np.array_equal(rows, dense_x)                   # I2 with the window excluded
    rows, _ = _all_groups_x(v, L, 1, k, k, "reuse", W)
    assert np.array_equal(rows, dense_x)                       # I3 with the window excluded
    for g in (2, 5):
        ref, _ = _all_groups_x(v, L, g, k, k + g - 1 + 2, "refine", W)
        for t in range(L):
            r = ref[t][ref[t] >= 0]
            assert np.all(r <= t - W) and len(r) == min(k, max(0, t - W + 1))


def _all_groups_x(v, L, g, k, C_, mode, W):
    G = (L + g - 1) // g
    return oracle.prefill_groups(v, L, g, k, C_, mode, np.arange(G), excl=W)


@pytest.mark.parametrize("W", [1, 4, 9])
def test_window_union_structure(case, W):
    L, k, inp, v, dense = case
    for mode, g in (("refine", 3), ("reuse", 4)):
        sel, _ = _all_groups(v, L, g, k, k + g + 1, mode)
        out = oracle.window_union(sel, np.arange(L), W)
        assert out.shape == (L, k + W)
        for t in range(L):
            lo = max(0, t - W + 1)
            r = out[t][out[t] >= 0]
            assert np.all(np.diff(r) > 0) and np.all(out[t][len(r):] == -1)
            s = sel[t][sel[t] >= 0]
            assert r.tolist() == s[s < lo].tolist() + list(range(lo, t + 1))
    # with the window excluded the union is disjoint: every k + W slot is used
    # once the prefix is long enough
    sel, _ = _all_groups_x(v, L, 2, k, L, "refine", W)
    out = oracle.window_union(sel, np.arange(L), W)
    for t in range(L):
        assert np.sum(out[t] >= 0) == min(k, max(0, t - W + 1)) + min(W, t + 1)
