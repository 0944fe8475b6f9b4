"""GPU parity on the float workloads at full size, in the launch configuration
the benchmark times.  Candidate sets and selections are checked with the tie
band of tests/parity.py; valid counts, order, padding and causality exactly;
the GPU's score of every selected position against the oracle's score of that
position (relative tolerance 1e-4 for bf16, the stated 2e-2 for fp8).

Sampling (the oracle computes any group on its own):
  * DSA-shaped prefill 16K (bf16, g=8): every one of the 2048 groups, Reuse and
    Refine; 256 dense rows in 64 strata;
  * long prefill 64K (fp8 e4m3, per-token scales, g=8): 64 groups (first two,
    last two, one seeded group in each of 60 strata), Reuse and Refine;
  * 128K prefill (bf16) for g in {4, 8, 16}: 64 groups each, Reuse and Refine;
    64 dense rows;
  * the MTP decode step (B=32, cache lengths in [32768, 131072], fp8): every
    sequence in all three modes.
Refine member rows are checked against the oracle's selection over the GPU's
candidate list, after that list is checked against the proxy's oracle scan
(so a candidate swap inside the proxy's tie band is accepted).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import top_token_selection_pivot_amd as pv
from parity import (EPS_BF16, EPS_FP8, check_band, check_row_shape, pmap, stratified_groups,
                    to_device)

pytestmark = pytest.mark.gpu


def _prefill_gpu(d, g, topk, C, mode):
    out, sc = pv.indexer(d["q"], d["w"], d["k"], g=g, topk=topk, C=C, mode=mode,
                         q_scale=d["q_scale"], k_scale=d["k_scale"], return_scores=True)
    cand = pv.candidates(d["q"], d["w"], d["k"], g=g, topk=topk, C=C, mode=mode,
                         q_scale=d["q_scale"], k_scale=d["k_scale"])
    torch.cuda.synchronize()
    return out, sc, cand


def _rows_of(t, groups, g, L):
    """Rows of the listed groups, copied to the host in one gather."""
    idx = np.concatenate([np.arange(j * g, min(L, j * g + g)) for j in groups])
    return t[torch.from_numpy(idx).to(t.device)].cpu().numpy()


def _check_groups(inp, d, g, topk, C, eps, groups, modes=("reuse", "refine")):
    """Reuse and Refine rows, scores and candidates of the listed groups."""
    v = oracle.View.of(inp)
    L = inp.L
    gpu = {}
    for mode in modes:
        out, sc, cand = _prefill_gpu(d, g, topk, C, mode)
        gi = torch.from_numpy(np.asarray(groups, np.int64)).to(cand.device)
        gpu[mode] = (_rows_of(out, groups, g, L), _rows_of(sc, groups, g, L),
                     cand[gi].cpu().numpy())
        del out, sc, cand
    starts = np.cumsum([0] + [min(g, L - j * g) for j in groups])

    def one(gi):
        j = groups[gi]
        first, last = j * g, min(L, j * g + g) - 1
        n = last - first + 1
        # the proxy's scan over its full prefix [0, last]
        _, _, psc = oracle.group(v, first, first, n, topk, C, "reuse")
        prefix = np.arange(last + 1)
        swaps = 0
        r0 = starts[gi]
        for mode in modes:
            rows, scores, cands = gpu[mode]
            m = C if mode == "refine" else topk
            c = cands[gi]
            swaps += check_band(c, prefix, psc, m, eps, f"{mode} candidates of group {j}")
            cv = c[c >= 0]
            for t in range(first, last + 1):
                r, s = rows[r0 + t - first], scores[r0 + t - first]
                pool = cv[cv <= t]
                if mode == "reuse":
                    assert r.tolist() == pool.tolist() + [-1] * (topk - len(pool)), (mode, t)
                    check_band(r[r >= 0], pool, psc[pool], len(pool), eps, f"reuse row {t}",
                               gpu_scores=s[:len(pool)])
                    assert np.all(np.isnan(s[len(pool):]))
                else:
                    sc = oracle.score_list(v, t, pool)
                    check_row_shape(r, min(topk, len(pool)), t)
                    swaps += check_band(r, pool, sc, topk, eps, f"refine row {t}", gpu_scores=s)
        return swaps

    swaps = sum(pmap(one, range(len(groups))))
    print(f"{modes}: {len(groups)} groups checked, {swaps} tie-band swaps", flush=True)


def _check_dense_rows(inp, d, topk, eps, rows):
    v = oracle.View.of(inp)
    out, sc = pv.indexer(d["q"], d["w"], d["k"], g=1, topk=topk, C=topk, mode="dense",
                         q_scale=d["q_scale"], k_scale=d["k_scale"], return_scores=True)
    torch.cuda.synchronize()
    ri = torch.from_numpy(np.asarray(rows, np.int64)).to(out.device)
    o, s = out[ri].cpu().numpy(), sc[ri].cpu().numpy()
    del out, sc

    def one(i):
        t = int(rows[i])
        ref = oracle.score_row(v, t, t + 1)
        check_row_shape(o[i], min(topk, t + 1), t)
        return check_band(o[i], np.arange(t + 1), ref, topk, eps, f"dense row {t}", gpu_scores=s[i])

    swaps = sum(pmap(one, range(len(rows))))
    print(f"dense: {len(rows)} rows checked, {swaps} tie-band swaps", flush=True)


def _stratified_rows(L, n, seed):
    rng = np.random.default_rng(seed)
    edges = np.linspace(0, L, n + 1).astype(np.int64)
    return sorted(set([0, 1, L - 2, L - 1] + [int(rng.integers(a, b)) for a, b in zip(edges[:-1], edges[1:])]))


@pytest.fixture(scope="module")
def dsa16k():
    inp = synth.make("dsa_prefill_16k")
    return inp, to_device(inp)


def test_dsa_prefill_16k_every_group(dsa16k):
    print("case: DSA-shaped prefill L=16384 H=64 D=128 g=8 k=2048 C=4096 bf16, all 2048 groups",
          flush=True)
    inp, d = dsa16k
    _check_groups(inp, d, 8, 2048, 4096, EPS_BF16, list(range(16384 // 8)))


def test_dsa_prefill_16k_dense_rows(dsa16k):
    print("case: DSA-shaped prefill L=16384 dense, 256 stratified rows", flush=True)
    inp, d = dsa16k
    _check_dense_rows(inp, d, 2048, EPS_BF16, _stratified_rows(16384, 252, 12))


def test_long_prefill_fp8_64k():
    print("case: long prefill fp8 L=65536 H=64 D=128 g=8 k=2048 C=4096, 64 groups", flush=True)
    inp = synth.make("long_prefill_fp8_64k")
    d = to_device(inp)
    _check_groups(inp, d, 8, 2048, 4096, EPS_FP8, stratified_groups(65536 // 8, 60, 3))


@pytest.fixture(scope="module")
def p128k():
    inp = synth.make("prefill_128k")
    return inp, to_device(inp)


@pytest.mark.parametrize("g", [8, 4, 16])
def test_prefill_128k(p128k, g):
    print(f"case: 128K prefill bf16 H=64 D=128 k=2048 C=4096 g={g}, 64 groups", flush=True)
    inp, d = p128k
    _check_groups(inp, d, g, 2048, 4096, EPS_BF16, stratified_groups(131072 // g, 60, 4 + g))


def test_prefill_128k_dense_rows(p128k):
    print("case: 128K prefill dense, 64 stratified rows", flush=True)
    inp, d = p128k
    _check_dense_rows(inp, d, 2048, EPS_BF16, _stratified_rows(131072, 60, 5))


def test_decode_mtp_b32_every_sequence():
    print("case: decode B=32 g=2 fp8 k=2048 C=4096, every sequence, three modes", flush=True)
    dec = synth.make("decode_mtp_b32")
    d = to_device(dec)
    topk, C = 2048, 4096
    gpu = {}
    for mode in ("refine", "reuse", "dense"):
        out, sc = pv.indexer_decode(d["q"], d["w"], d["k"], d["cache_len"], topk=topk, C=C,
                                    mode=mode, q_scale=d["q_scale"], k_scale=d["k_scale"],
                                    return_scores=True)
        cand = None
        if mode != "dense":
            cand = pv.decode_candidates(d["q"], d["w"], d["k"], d["cache_len"], topk=topk, C=C,
                                        mode=mode, q_scale=d["q_scale"],
                                        k_scale=d["k_scale"]).cpu().numpy()
        torch.cuda.synchronize()
        gpu[mode] = (out.cpu().numpy(), sc.cpu().numpy(), cand)

    def one(b):
        v = oracle.decode_view(dec, b)
        n = int(dec.cache_len[b])
        _, _, psc = oracle.group(v, 0, n - 2, 2, topk, C, "reuse")
        swaps = 0
        for mode, (out, scores, cands) in gpu.items():
            for i in range(2):
                t = n - 2 + i
                r, s = out[b, i], scores[b, i]
                if mode == "dense":
                    sc = oracle.score_row(v, i, t + 1)
                    swaps += check_band(r, np.arange(t + 1), sc, topk, EPS_FP8,
                                        f"dense seq {b} member {i}", gpu_scores=s)
                    continue
                m = C if mode == "refine" else topk
                c = cands[b]
                if i == 0:
                    swaps += check_band(c, np.arange(n), psc, m, EPS_FP8, f"{mode} cand seq {b}")
                cv = c[c >= 0]
                pool = cv[cv <= t]
                if mode == "reuse":
                    assert r.tolist() == pool.tolist() + [-1] * (topk - len(pool))
                    check_band(r[r >= 0], pool, psc[pool], len(pool), EPS_FP8, f"reuse seq {b}",
                               gpu_scores=s[:len(pool)])
                    assert np.all(np.isnan(s[len(pool):]))
                else:
                    sc = oracle.score_list(v, i, pool)
                    swaps += check_band(r, pool, sc, topk, EPS_FP8, f"refine seq {b} member {i}",
                                        gpu_scores=s)
        return swaps

    swaps = sum(pmap(one, range(dec.B)))
    print(f"decode: 32 sequences x 3 modes checked, {swaps} tie-band swaps", flush=True)


def _check_window_rows(rows, positions, W, topk, excluded):
    """Rows with a sliding window: the selection's entries below the window,
    then every position of the window, then -1; with the window excluded the
    selection holds min(topk, t-W+1) entries (dense and Refine)."""
    sel = []
    for r, t in zip(rows, positions):
        lo = max(0, int(t) - W + 1)
        valid = r[r >= 0]
        assert np.all(np.diff(valid) > 0) and np.all(r[len(valid):] == -1), t
        s = valid[valid < lo]
        assert valid[len(s):].tolist() == list(range(lo, int(t) + 1)), t
        if excluded:
            assert len(s) == min(topk, max(0, int(t) - W + 1)), t
        sel.append(np.concatenate([s, np.full(topk - len(s), -1)]))
    return np.array(sel)


def test_window_16k_and_decode(dsa16k):
    print("case: window 128 (shared, excluded) at the 16K prefill and the B=32 decode step",
          flush=True)
    W, topk = 128, 2048
    inp, d = dsa16k
    v = oracle.View.of(inp)
    L = inp.L
    kw = dict(g=8, topk=topk, C=4096, mode="refine")
    plain = pv.indexer(d["q"], d["w"], d["k"], **kw).cpu().numpy()
    shared = pv.indexer(d["q"], d["w"], d["k"], window=W, window_mode="shared", **kw).cpu().numpy()
    # the shared window leaves the selection as it is: exactly the union
    assert np.array_equal(shared, oracle.window_union(plain, np.arange(L), W))
    excl = pv.indexer(d["q"], d["w"], d["k"], window=W, window_mode="excluded", **kw).cpu().numpy()
    _check_window_rows(excl, np.arange(L), W, topk, True)
    dx = pv.indexer(d["q"], d["w"], d["k"], g=1, topk=topk, C=topk, mode="dense", window=W,
                    window_mode="excluded").cpu().numpy()
    rows = [0, 127, 128, 2175, 9000, 16383]
    sel = _check_window_rows(dx[rows], rows, W, topk, True)
    for r, t in zip(sel, rows):
        n = max(0, t - W + 1)
        sc = oracle.score_row(v, t, n) if n else np.zeros(0)
        check_band(r, np.arange(n), sc, topk, EPS_BF16, f"dense window-excluded row {t}")

    dec = synth.make("decode_mtp_b32")
    d = to_device(dec)
    pos = (dec.cache_len[:, None] - 2 + np.arange(2)[None, :]).reshape(-1)
    dkw = dict(topk=topk, C=4096, q_scale=d["q_scale"], k_scale=d["k_scale"])
    for mode in ("refine", "dense"):
        plain = pv.indexer_decode(d["q"], d["w"], d["k"], d["cache_len"], mode=mode, **dkw)
        shared = pv.indexer_decode(d["q"], d["w"], d["k"], d["cache_len"], mode=mode, window=W,
                                   window_mode="shared", **dkw)
        plain = plain.cpu().numpy().reshape(-1, topk)
        assert np.array_equal(shared.cpu().numpy().reshape(-1, topk + W),
                              oracle.window_union(plain, pos, W))
        ex = pv.indexer_decode(d["q"], d["w"], d["k"], d["cache_len"], mode=mode, window=W,
                               window_mode="excluded", **dkw).cpu().numpy().reshape(-1, topk + W)
        sel = _check_window_rows(ex, pos, W, topk, True)
        if mode == "dense":
            for b in (0, 31):
                vb = oracle.decode_view(dec, b)
                for i in range(2):
                    t = int(pos[2 * b + i])
                    n = t - W + 1
                    sc = oracle.score_row(vb, i, n)
                    check_band(sel[2 * b + i], np.arange(n), sc, topk, EPS_FP8,
                               f"decode dense window-excluded seq {b}")


def test_score_rows_16k_sampled(dsa16k):
    """The score-row export (the scan kernel's own rows) against the oracle's
    scores: dense rows and proxy rows of the 16K workload, every key, within
    1e-4 of the score plus 1e-4 of the row's mean magnitude (binary32 sums of
    D products whose terms may cancel)."""
    print("case: score rows of the 16K prefill (dense and proxy rows)", flush=True)
    inp, d = dsa16k
    v = oracle.View.of(inp)
    rows = [0, 1, 777, 8191, 16383]
    for t in rows:
        s = pv.score_rows(d["q"], d["w"], d["k"], row_begin=t, row_end=t + 1)[0].cpu().numpy()
        ref = oracle.score_row(v, t, t + 1)
        assert np.all(np.isnan(s[t + 1:]))
        assert np.all(np.abs(s[:t + 1] - ref) <= EPS_BF16 * (np.abs(ref) + np.abs(ref).mean()))
    qbar, qs, wbar = pv.proxy_mean(d["q"], d["w"], 8)
    for j in (0, 1000, 2047):
        s = pv.score_rows(qbar, wbar, d["k"], row_begin=j, row_end=j + 1, pos_mul=8,
                          pos_add=7)[0].cpu().numpy()
        pq, _, pw = oracle.proxy(v, j * 8, 8)
        pv_ = oracle.View("bf16", pq[None], None, pw[None], inp.k, None)
        e = j * 8 + 7
        ref = oracle.score_row(pv_, 0, e + 1)
        assert np.all(np.isnan(s[e + 1:]))
        assert np.all(np.abs(s[:e + 1] - ref) <= EPS_BF16 * (np.abs(ref) + np.abs(ref).mean()))
