"""Helpers that compare GPU indexer outputs with the CPU oracle.

Exact comparison (integer-valued inputs, where every binary32 sum is exact):
rows must be identical.  Float inputs: the GPU accumulates in binary32 while the
oracle sums in double, so two keys whose exact scores differ by less than the
accumulation error may swap places at the selection threshold.  The tie band
accepts exactly those swaps: with tau the m-th largest oracle score of the
pool, every position the GPU picked that the oracle did not must score at
least tau - eps*|tau|, and every position the oracle picked that the GPU did
not must score at most tau + eps*|tau|; the number of selected positions must
match exactly.  Scores the GPU reports for its selected positions must agree
with the oracle's score of the same position: |s_gpu - s_orc| <=
eps * max(|s_orc|, |tau|); entries past the selection are NaN.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle

# bf16 float inputs: about 100x the binary32 accumulation error over D=128
# products and H=64 heads ((D + H) * 2^-24 ~ 1.1e-5 of the absolute sum).
EPS_BF16 = 1e-4
# fp8 inputs: the stated score tolerance.
EPS_FP8 = 2e-2

# host threads for the oracle (its C calls release the interpreter lock); at
# most 16, the host share of one GPU
THREADS = max(1, min(16, os.cpu_count() or 1))


def pmap(fn, items):
    """fn over items on THREADS host threads, results in order."""
    items = list(items)
    if THREADS == 1 or len(items) < 2:
        return [fn(x) for x in items]
    with ThreadPoolExecutor(THREADS) as ex:
        return list(ex.map(fn, items))


def stratified_groups(G: int, n_extra: int, seed: int):
    """The first two and last two groups plus one seeded group from each of
    n_extra equal strata of the rest, so every part of the sequence (every
    workspace pass and scan launch) is sampled."""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, G - 2, G - 1]
    if G <= 4 + n_extra:
        return list(range(G))
    edges = np.linspace(2, G - 2, n_extra + 1).astype(np.int64)
    extra = [int(rng.integers(lo, hi)) for lo, hi in zip(edges[:-1], edges[1:]) if hi > lo]
    return sorted(set(fixed + extra))


def to_device(inp, device="cuda"):
    """Upload PrefillInputs / DecodeInputs codes as device tensors (bf16 or fp8)."""
    def codes(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(a).view(torch.float8_e4m3fn).to(device)

    def f32(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)

    d = dict(q=codes(inp.q), w=f32(inp.w), k=codes(inp.k), q_scale=f32(inp.q_scale),
             k_scale=f32(inp.k_scale))
    if hasattr(inp, "cache_len"):
        d["cache_len"] = torch.from_numpy(inp.cache_len.astype(np.int32)).to(device)
    return d


def check_row_shape(row, n_valid_expected, t=None):
    row = np.asarray(row)
    valid = row[row >= 0]
    assert len(valid) == n_valid_expected, (len(valid), n_valid_expected)
    assert np.all(row[len(valid):] == -1), "-1 padding must be at the tail"
    assert np.all(np.diff(valid) > 0), "positions must be strictly ascending"
    if t is not None:
        assert np.all(valid <= t), "a future position was selected"


def check_scores(gpu_row, gpu_scores, pos_score, eps, tau, what=""):
    """GPU scores of the selected positions against the oracle's scores of the
    same positions (pos_score: array aligned with the valid entries)."""
    gpu_row = np.asarray(gpu_row)
    gs = np.asarray(gpu_scores, np.float64)
    nv = int((gpu_row >= 0).sum())
    assert np.all(np.isnan(gs[nv:])), f"{what}: scores past the selection must be NaN"
    if nv == 0:
        return
    got = gs[:nv]
    ref = np.asarray(pos_score, np.float64)
    tol = eps * np.maximum(np.abs(ref), abs(tau))
    bad = np.abs(got - ref) > tol
    assert not bad.any(), (f"{what}: score of position {gpu_row[:nv][bad][0]}: GPU {got[bad][0]!r}, "
                           f"oracle {ref[bad][0]!r}")


def check_band(gpu_row, pool_pos, pool_scores, m, eps, what="", gpu_scores=None):
    """gpu_row: selected positions (ascending, -1 padded) out of pool_pos whose
    oracle scores are pool_scores; gpu_scores (optional): the GPU's scores of
    its selected positions.  Returns the number of tie-band swaps."""
    pool_pos = np.asarray(pool_pos, np.int64)
    pool_scores = np.asarray(pool_scores, np.float64)
    n = len(pool_pos)
    r = min(m, n)
    gpu_row = np.asarray(gpu_row)
    check_row_shape(gpu_row, r)
    g = gpu_row[gpu_row >= 0].astype(np.int64)
    order = np.argsort(pool_pos, kind="stable")
    sp = pool_pos[order]
    ss = pool_scores[order]
    at = np.searchsorted(sp, g)
    inpool = (at < n) & (sp[np.minimum(at, max(n - 1, 0))] == g) if n else np.zeros(len(g), bool)
    assert inpool.all(), f"{what}: position {g[~inpool][0]} outside the pool"
    gsc = ss[at] if n else np.zeros(0)
    tau = float(np.partition(pool_scores, n - r)[n - r]) if r > 0 else 0.0
    if gpu_scores is not None:
        check_scores(gpu_row, gpu_scores, gsc, eps, tau, what)
    if r == 0:
        return 0
    ref = oracle.topk(pool_scores, m, pool_pos.astype(np.int32))
    o = ref[ref >= 0].astype(np.int64)
    if np.array_equal(g, o):
        return 0
    band = eps * max(abs(tau), 1e-30)
    extra = np.setdiff1d(g, o)
    missing = np.setdiff1d(o, g)
    esc = ss[np.searchsorted(sp, extra)]
    msc = ss[np.searchsorted(sp, missing)]
    assert np.all(esc >= tau - band), f"{what}: GPU picked {extra[esc < tau - band][0]} below tau {tau}"
    assert np.all(msc <= tau + band), f"{what}: GPU dropped {missing[msc > tau + band][0]} above tau {tau}"
    return len(extra)
