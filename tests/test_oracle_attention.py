"""Pins of the oracle's sparse main attention (tutorial "Sparse Attention의
Indexer", text after Figure 1: softmax over the selected positions only, values
combined with those weights) against facts that do not come from the oracle:
PyTorch's scaled dot-product attention (float64, causal) when every position is
selected, closed forms (one selected position; a zero query averages the
selected values, exact rationals) and invariances.  CPU only."""
from fractions import Fraction

import numpy as np
import torch

import oracle
import synth


def _bf16(rng, shape, lo=-3, hi=4, div=4.0):
    return synth.encode_bf16(rng.integers(lo, hi, shape).astype(np.float32) / div)


def _val(codes):
    return (codes.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_all_positions_equal_causal_sdpa():
    rng = np.random.default_rng(1)
    L, Hq, d, dv = 40, 4, 16, 8
    q, k, v = _bf16(rng, (L, Hq, d)), _bf16(rng, (L, d)), _bf16(rng, (L, dv))
    idx = np.array([[s if s <= t else -1 for s in range(L)] for t in range(L)], np.int32)
    got = oracle.sparse_attention(q, k, v, idx)
    qt = torch.from_numpy(_val(q)).permute(1, 0, 2)          # [Hq, L, d]
    kt = torch.from_numpy(_val(k))[None].expand(Hq, L, d)   # one key row shared by the heads
    vt = torch.from_numpy(_val(v))[None].expand(Hq, L, dv)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    assert np.allclose(got, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_one_selected_position_returns_its_value_row():
    rng = np.random.default_rng(2)
    q, k, v = _bf16(rng, (5, 3, 8)), _bf16(rng, (30, 8)), _bf16(rng, (30, 6))
    idx = np.full((5, 7), -1, np.int32)
    for r in range(5):
        idx[r, r + 1] = 3 * r + 2
    got = oracle.sparse_attention(q, k, v, idx)
    for r in range(5):
        assert np.array_equal(got[r], np.broadcast_to(_val(v)[3 * r + 2], (3, 6)))


def test_zero_query_averages_the_selected_values_exactly():
    rng = np.random.default_rng(3)
    q = synth.encode_bf16(np.zeros((2, 2, 8), np.float32))
    k, v = _bf16(rng, (20, 8)), _bf16(rng, (20, 4))
    idx = np.array([[0, 5, 7, 19], [3, 3, -1, 11]], np.int32)  # a repeated position counts twice
    got = oracle.sparse_attention(q, k, v, idx)
    vf = _val(v)
    for r in range(2):
        sel = [s for s in idx[r] if s >= 0]
        for c in range(4):
            mean = sum(Fraction(float(vf[s, c])) for s in sel) / len(sel)
            assert got[r, 0, c] == float(mean) and got[r, 1, c] == float(mean)


def test_padding_order_and_range_do_not_matter():
    rng = np.random.default_rng(4)
    q, k, v = _bf16(rng, (6, 2, 8)), _bf16(rng, (50, 8)), _bf16(rng, (50, 8))
    base = np.array([rng.choice(50, 9, replace=False) for _ in range(6)], np.int32)
    ref = oracle.sparse_attention(q, k, v, base)
    shuffled = np.array([rng.permutation(r) for r in base], np.int32)
    padded = np.concatenate([shuffled, np.full((6, 3), -1, np.int32), np.full((6, 2), 50, np.int32)], 1)
    got = oracle.sparse_attention(q, k, v, padded, seq_len=50)
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13)
    empty = oracle.sparse_attention(q, k, v, np.full((6, 4), -1, np.int32))
    assert np.all(empty == 0)


def test_decode_layout_reads_each_sequence():
    rng = np.random.default_rng(5)
    B, S, g, Hq, d, dv = 3, 25, 2, 2, 8, 8
    q, k, v = _bf16(rng, (B * g, Hq, d)), _bf16(rng, (B, S, d)), _bf16(rng, (B, S, dv))
    idx = rng.integers(-1, S, (B * g, 6)).astype(np.int32)
    got = oracle.sparse_attention(q, k, v, idx, rows_per_seq=g)
    for b in range(B):
        one = oracle.sparse_attention(q[b * g:(b + 1) * g], k[b], v[b], idx[b * g:(b + 1) * g])
        assert np.array_equal(got[b * g:(b + 1) * g], one)
