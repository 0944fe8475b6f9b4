"""GPU parity of the sparse main attention over the selected positions
(tutorial "Sparse Attention의 Indexer", text after Figure 1) against the
oracle, which computes in double.  The GPU sums in binary32 and feeds the
softmax weights to the matrix cores as two bf16 terms, so each output agrees
with the oracle to within 1e-4 of the row's largest value magnitude, plus 1e-4
relative; the bound is derived in the design notes (scores exact to binary32
rounding over d = 128 products, weights split to about 2^-17, sums over at
most a few thousand terms)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import top_token_selection_pivot_amd as pv

pytestmark = pytest.mark.gpu


def _codes(rng, shape, scale=1.0):
    return synth.encode_bf16((rng.standard_normal(shape) * scale).astype(np.float32))


def _t(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _close(got, ref, what):
    vmax = np.abs(ref).max(axis=-1, keepdims=True).max(axis=-2, keepdims=True)
    err = np.abs(got - ref)
    bound = 1e-4 * np.maximum(vmax, 1e-30) + 1e-4 * np.abs(ref)
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} values off, worst {(err / np.maximum(bound, 1e-30)).max():.2f}x the bound"


def _sets(rng, R, nkeys, nidx, limit=None, pad=0.0):
    """Ascending positions per row (an indexer's rows), -1 padded."""
    out = np.full((R, nidx), -1, np.int32)
    for r in range(R):
        hi = nkeys if limit is None else min(nkeys, limit[r] + 1)
        n = min(nidx, hi, int(nidx * (1 - pad * rng.random())))
        out[r, :n] = np.sort(rng.choice(hi, n, replace=False))
    return out


@pytest.mark.parametrize("Hq", [32, 64])
def test_attention_few_rows_chunked(Hq):
    # few rows: every row's slots are split over several waves and merged
    print(f"case: sparse attention R=300 Hq={Hq} nidx=700 (chunked)", flush=True)
    rng = np.random.default_rng(Hq)
    L = 3000
    q, k, v = _codes(rng, (300, Hq, 128)), _codes(rng, (L, 128)), _codes(rng, (L, 128))
    idx = _sets(rng, 300, L, 700, pad=0.5)
    idx[3] = -1                         # an empty row
    idx[4, :5] = [7, 7, 7, -1, 2999]    # repeats count each time
    got = pv.sparse_attention(_t(q), _t(k), _t(v), _t(idx)).cpu().numpy()
    ref = oracle.sparse_attention(q, k, v, idx)
    assert np.all(got[3] == 0)
    _close(got, ref, "chunked")


@pytest.mark.parametrize("Hq", [32, 64])
def test_attention_merge_over_many_chunks(Hq):
    # 3 rows of 4100 slots: 33 chunks each, merged 16 at a time; row 1 has no
    # valid slot in its first 2100 entries, row 2 none after its first 1000
    print(f"case: sparse attention R=3 Hq={Hq} nidx=4100 (33 chunks)", flush=True)
    rng = np.random.default_rng(100 + Hq)
    L = 5000
    q, k, v = _codes(rng, (3, Hq, 128)), _codes(rng, (L, 128)), _codes(rng, (L, 128))
    idx = rng.integers(0, L, (3, 4100)).astype(np.int32)
    idx[1, :2100] = -1
    idx[2, 1000:] = -1
    idx[2, 3000] = L + 7  # outside the sequence: skipped
    got = pv.sparse_attention(_t(q), _t(k), _t(v), _t(idx)).cpu().numpy()
    ref = oracle.sparse_attention(q, k, v, idx)
    _close(got, ref, "33 chunks")


def test_attention_many_rows_single_chunk():
    # many rows: one wave per row, no merge; causal rows like an indexer's output
    print("case: sparse attention R=1100 Hq=64 nidx=300 (one chunk per row)", flush=True)
    rng = np.random.default_rng(7)
    L = 1100
    q, k, v = _codes(rng, (L, 64, 128)), _codes(rng, (L, 128)), _codes(rng, (L, 128))
    idx = _sets(rng, L, L, 300, limit=np.arange(L))
    got = pv.sparse_attention(_t(q), _t(k), _t(v), _t(idx)).cpu().numpy()
    ref = oracle.sparse_attention(q, k, v, idx)
    _close(got, ref, "single chunk")


def test_attention_decode_layout_and_range():
    print("case: sparse attention decode layout B=6 g=2 S=2500 Hq=64 nidx=1000", flush=True)
    rng = np.random.default_rng(9)
    B, g, S = 6, 2, 2500
    q = _codes(rng, (B * g, 64, 128))
    k, v = _codes(rng, (B, S, 128)), _codes(rng, (B, S, 128))
    seq_len = 2400  # positions 2400.. of each sequence are outside the range
    idx = _sets(rng, B * g, S, 1000, pad=0.3)
    got = pv.sparse_attention(_t(q), _t(k), _t(v), _t(idx), rows_per_seq=g,
                              seq_len=seq_len).cpu().numpy()
    ref = oracle.sparse_attention(q, k, v, idx, rows_per_seq=g, seq_len=seq_len)
    _close(got, ref, "decode layout")


def test_attention_large_scores_and_full_selection():
    # scores in the thousands: the running maximum keeps the exponentials finite;
    # every position 0..t selected: causal dense attention
    print("case: sparse attention, large scores and full causal selection", flush=True)
    rng = np.random.default_rng(11)
    L = 500
    q, k, v = _codes(rng, (L, 32, 128), 4.0), _codes(rng, (L, 128), 4.0), _codes(rng, (L, 128))
    idx = np.array([[s if s <= t else -1 for s in range(L)] for t in range(L)], np.int32)
    for scale in (1.0, 1.0 / np.sqrt(128)):
        got = pv.sparse_attention(_t(q), _t(k), _t(v), _t(idx), scale=scale).cpu().numpy()
        ref = oracle.sparse_attention(q, k, v, idx, scale=scale)
        assert np.isfinite(got).all()
        _close(got, ref, f"scale {scale}")


def test_attention_score_ramps():
    # the score of position s is k_s[0] = 0.05 s, plus 20 from s = 1000 on:
    # read in ascending order a head's maximum creeps up (several tiles pass
    # before it has moved far enough to rescale) and jumps once; read in
    # descending order the first tile holds the maximum
    print("case: sparse attention, rising, falling and jumping score ramps", flush=True)
    rng = np.random.default_rng(17)
    L, Hq = 2048, 64
    kf = rng.standard_normal((L, 128)).astype(np.float32)
    kf[:, 0] = 0.05 * np.arange(L) + 20.0 * (np.arange(L) >= 1000)
    qf = np.zeros((4, Hq, 128), np.float32)
    qf[:, :, 0] = 1.0
    qf[3, :, 0] = np.linspace(0.1, 1.0, Hq)  # a different slope per head
    q, k, v = synth.encode_bf16(qf), synth.encode_bf16(kf), _codes(rng, (L, 128))
    idx = np.stack([np.arange(L), np.arange(L)[::-1], rng.permutation(L), np.arange(L)]).astype(np.int32)
    got = pv.sparse_attention(_t(q), _t(k), _t(v), _t(idx), scale=1.0).cpu().numpy()
    ref = oracle.sparse_attention(q, k, v, idx, scale=1.0)
    _close(got, ref, "ramps")
    many = np.repeat(idx, 300, axis=0)  # 1200 rows: one chunk per row, no merge
    got = pv.sparse_attention(_t(np.repeat(q, 300, axis=0)), _t(k), _t(v), _t(many), scale=1.0).cpu().numpy()
    _close(got[::300], ref, "ramps, one chunk per row")


def test_attention_after_the_indexer():
    # the indexer's own rows (Refine with a shared window) feed the attention
    print("case: indexer rows (Refine g=4, window 16) -> sparse attention", flush=True)
    inp = synth.tiny_integer(L=2048, H=4, D=32, seed=1001)
    d = {"q": _t(inp.q), "w": _t(inp.w), "k": _t(inp.k)}
    rows = pv.indexer(d["q"], d["w"], d["k"], g=4, topk=64, C=256, mode="refine", window=16)
    rng = np.random.default_rng(13)
    q, k, v = _codes(rng, (2048, 64, 128)), _codes(rng, (2048, 128)), _codes(rng, (2048, 128))
    got = pv.sparse_attention(_t(q), _t(k), _t(v), rows).cpu().numpy()
    ref = oracle.sparse_attention(q, k, v, rows.cpu().numpy())
    _close(got, ref, "after the indexer")
