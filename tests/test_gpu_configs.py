"""GPU parity on the float workloads at full size (sampled rows), in the launch
configuration the benchmark times.  Candidate sets and selections are checked
with the tie band of tests/parity.py; valid counts, order, padding and
causality are checked exactly.

Workloads: DSA-shaped prefill 16K (bf16), long prefill 64K (fp8 e4m3 with
per-token scales), 128K prefill (bf16; g in {4, 8, 16}) and the MTP decode step
(B=32, cache lengths in [32768, 131072], fp8).  Sampled groups: the first two,
the last two and seeded others.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import top_token_selection_pivot_amd as pv
from parity import EPS_BF16, EPS_FP8, check_band, check_row_shape, to_device

pytestmark = pytest.mark.gpu


def _sample_groups(G, n_extra, seed):
    rng = np.random.default_rng(seed)
    extra = rng.choice(np.arange(2, G - 2), size=n_extra, replace=False) if G > 4 + n_extra else []
    return sorted(set([0, 1, G - 2, G - 1] + list(map(int, extra))))


def _check_groups(inp, d, g, topk, C, eps, groups, modes=("reuse", "refine")):
    v = oracle.View.of(inp)
    L = inp.L
    for mode in modes:
        m = C if mode == "refine" else topk
        out = pv.indexer(d["q"], d["w"], d["k"], g=g, topk=topk, C=C, mode=mode,
                         q_scale=d["q_scale"], k_scale=d["k_scale"])
        cand = pv.candidates(d["q"], d["w"], d["k"], g=g, topk=topk, C=C, mode=mode,
                             q_scale=d["q_scale"], k_scale=d["k_scale"])
        torch.cuda.synchronize()
        swaps = 0
        for j in groups:
            first, last = j * g, min(L, j * g + g) - 1
            rows = out[first:last + 1].cpu().numpy()
            c = cand[j].cpu().numpy()
            _, _, psc = oracle.group(v, first, first, last - first + 1, topk, C, mode)
            # the proxy's top-m over its full prefix [0, last]
            swaps += check_band(c, np.arange(last + 1), psc, m, eps, f"{mode} cand g{j}")
            cv = c[c >= 0]
            for t in range(first, last + 1):
                r = rows[t - first]
                if mode == "reuse":
                    exp = cv[cv <= t]
                    assert r.tolist() == exp.tolist() + [-1] * (topk - len(exp)), (mode, t)
                else:
                    pool = cv[cv <= t]
                    sc = oracle.score_pairs(v, np.full(len(pool), t), pool)
                    check_row_shape(r, min(topk, len(pool)), t)
                    swaps += check_band(r, pool, sc, topk, eps, f"{mode} row {t}")
        print(f"{mode}: {len(groups)} groups checked, {swaps} tie-band swaps", flush=True)


def _check_dense_rows(inp, d, topk, eps, rows):
    v = oracle.View.of(inp)
    out = pv.indexer(d["q"], d["w"], d["k"], g=1, topk=topk, C=topk, mode="dense",
                     q_scale=d["q_scale"], k_scale=d["k_scale"])
    torch.cuda.synchronize()
    for t in rows:
        sc = oracle.score_row(v, int(t), int(t) + 1)
        check_band(out[t].cpu().numpy(), np.arange(t + 1), sc, topk, eps, f"dense row {t}")
    return out


def test_dsa_prefill_16k():
    print("case: DSA-shaped prefill L=16384 H=64 D=128 g=8 k=2048 C=4096 bf16", flush=True)
    inp = synth.make("dsa_prefill_16k")
    d = to_device(inp)
    G = 16384 // 8
    _check_groups(inp, d, 8, 2048, 4096, EPS_BF16, _sample_groups(G, 4, 2))
    _check_dense_rows(inp, d, 2048, EPS_BF16, [0, 2047, 2048, 9000, 16383])


def test_long_prefill_fp8_64k():
    print("case: long prefill fp8 L=65536 H=64 D=128 g=8 k=2048 C=4096", flush=True)
    inp = synth.make("long_prefill_fp8_64k")
    d = to_device(inp)
    _check_groups(inp, d, 8, 2048, 4096, EPS_FP8, _sample_groups(65536 // 8, 2, 3))


def test_prefill_128k():
    print("case: 128K prefill bf16 H=64 D=128 k=2048 C=4096, g in {8, 4, 16}", flush=True)
    inp = synth.make("prefill_128k")
    d = to_device(inp)
    L = 131072
    _check_groups(inp, d, 8, 2048, 4096, EPS_BF16, _sample_groups(L // 8, 2, 4),
                  modes=("refine",))
    for g in (4, 16):
        _check_groups(inp, d, g, 2048, 2 * 2048, EPS_BF16, [L // g - 1, 777], modes=("refine",))
    _check_dense_rows(inp, d, 2048, EPS_BF16, [4095, 131071])


def test_decode_mtp_b32():
    print("case: decode B=32 g=2 fp8 k=2048 C=4096, cache lengths in [32768, 131072]", flush=True)
    dec = synth.make("decode_mtp_b32")
    d = to_device(dec)
    for mode in ("refine", "reuse", "dense"):
        out = pv.indexer_decode(d["q"], d["w"], d["k"], d["cache_len"], topk=2048, C=4096,
                                mode=mode, q_scale=d["q_scale"], k_scale=d["k_scale"])
        torch.cuda.synchronize()
        out = out.cpu().numpy()
        for b in range(32):  # shape, order and causality of every row
            n = int(dec.cache_len[b])
            for i in range(2):
                t = n - 2 + i
                exp = min(2048, t + 1)
                if mode == "reuse":
                    exp = np.sum((out[b, 1] >= 0) & (out[b, 1] <= t))
                check_row_shape(out[b, i], exp, t)
        for b in (0, 7, 31):
            v = oracle.decode_view(dec, b)
            n = int(dec.cache_len[b])
            ref, cand, psc = oracle.decode_seq(dec, b, 2048, 4096, mode)
            if mode == "dense":
                for i in range(2):
                    t = n - 2 + i
                    sc = oracle.score_row(v, i, t + 1)
                    check_band(out[b, i], np.arange(t + 1), sc, 2048, EPS_FP8, f"dense seq {b}")
                continue
            m = 4096 if mode == "refine" else 2048
            c = pv.decode_candidates(d["q"], d["w"], d["k"], d["cache_len"], topk=2048, C=4096,
                                     mode=mode, q_scale=d["q_scale"],
                                     k_scale=d["k_scale"])[b].cpu().numpy()
            check_band(c, np.arange(n), psc, m, EPS_FP8, f"{mode} cand seq {b}")
            cv = c[c >= 0]
            for i in range(2):
                t = n - 2 + i
                r = out[b, i]
                if mode == "reuse":
                    exp = cv[cv <= t]
                    assert r.tolist() == exp.tolist() + [-1] * (2048 - len(exp))
                else:
                    pool = cv[cv <= t]
                    sc = oracle.score_pairs(v, np.full(len(pool), i), pool)
                    check_band(r, pool, sc, 2048, EPS_FP8, f"refine seq {b} member {i}")
        print(f"decode {mode}: ok", flush=True)


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


def test_window_16k_and_decode():
    print("case: window 128 (shared, excluded) at the 16K prefill and the B=32 decode step",
          flush=True)
    W, topk = 128, 2048
    inp = synth.make("dsa_prefill_16k")
    d = to_device(inp)
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
