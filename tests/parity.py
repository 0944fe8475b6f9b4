"""Helpers that compare GPU indexer outputs with the CPU oracle.

Exact comparison (integer-valued inputs, where every binary32 sum is exact):
rows must be identical.  Float inputs: the GPU accumulates in binary32 while the
oracle sums in double, so two keys whose exact scores differ by less than the
accumulation error may swap places at the selection threshold.  The tie band
accepts exactly those swaps: with tau the m-th largest oracle score of the
pool, every position the GPU picked that the oracle did not must score at
least tau - eps*|tau|, and every position the oracle picked that the GPU did
not must score at most tau + eps*|tau|; the number of selected positions must
match exactly.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

# bf16 float inputs: about 100x the binary32 accumulation error over D=128
# products and H=64 heads ((D + H) * 2^-24 ~ 1.1e-5 of the absolute sum).
EPS_BF16 = 1e-4
# fp8 inputs: the stated score tolerance.
EPS_FP8 = 2e-2


def to_device(inp, device="cuda"):
    """Upload PrefillInputs / DecodeInputs codes as raw device tensors."""
    def codes(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

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


def check_band(gpu_row, pool_pos, pool_scores, m, eps, what=""):
    """gpu_row: selected positions (ascending, -1 padded) out of pool_pos whose
    oracle scores are pool_scores."""
    pool_pos = np.asarray(pool_pos, np.int64)
    pool_scores = np.asarray(pool_scores, np.float64)
    n = len(pool_pos)
    r = min(m, n)
    gpu_row = np.asarray(gpu_row)
    check_row_shape(gpu_row, r)
    g = set(gpu_row[gpu_row >= 0].tolist())
    ref = oracle.topk(pool_scores, m, pool_pos.astype(np.int32))
    o = set(ref[ref >= 0].tolist())
    assert g <= set(pool_pos.tolist()), f"{what}: position outside the pool"
    if g == o:
        return 0
    score = dict(zip(pool_pos.tolist(), pool_scores.tolist()))
    tau = np.sort(pool_scores)[::-1][r - 1]
    band = eps * max(abs(tau), 1e-30)
    for x in g - o:
        assert score[x] >= tau - band, f"{what}: GPU picked {x} ({score[x]}) below tau {tau}"
    for x in o - g:
        assert score[x] <= tau + band, f"{what}: GPU dropped {x} ({score[x]}) above tau {tau}"
    return len(g - o)
