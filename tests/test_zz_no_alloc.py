"""The allocation-free decode entry point (pivot_indexer_decode_noalloc) gives
exactly what pivot_indexer_decode gives with a caller workspace: two calls in a
row through the C ABI, the second with a smaller input, in every mode, indices
and scores bit for bit; and a step too large for its scratch array is refused
with PIVOT_ERR_WORKSPACE before anything runs."""
import numpy as np
import pytest
import torch

import oracle
import synth
import top_token_selection_pivot_amd as pv
from parity import to_device

pytestmark = pytest.mark.gpu


def _small_integer_decode(B, lens, g, H, D, Lmax, seed):
    rng = np.random.default_rng(seed)
    qf = rng.integers(-2, 3, (B, g, H, D)).astype(np.float32)
    kf = rng.integers(-2, 3, (B, Lmax, D)).astype(np.float32)
    w = rng.integers(1, 4, (B, g, H)).astype(np.float32)
    return synth.DecodeInputs("bf16", B, Lmax, H, D, g, synth.encode_bf16(qf), None, w,
                              synth.encode_bf16(kf), None, np.asarray(lens, np.int32))


def _both(d, B, g, topk, C, mode):
    ref, ref_s = pv.indexer_decode(d["q"], d["w"], d["k"], d["cache_len"], topk=topk, C=C, mode=mode,
                                   q_scale=d["q_scale"], k_scale=d["k_scale"], return_scores=True)
    out = torch.full((B, g, topk), 7, dtype=torch.int32, device="cuda")
    sc = torch.full((B, g, topk), 3.0, dtype=torch.float32, device="cuda")
    pv.indexer_decode_noalloc(d["q"], d["w"], d["k"], d["cache_len"], topk=topk, C=C, mode=mode,
                              q_scale=d["q_scale"], k_scale=d["k_scale"], out=out, out_scores=sc)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), ref_s.cpu().numpy(), out.cpu().numpy(), sc.cpu().numpy()


def _same(a, b):
    return np.array_equal(np.nan_to_num(a, nan=-7.0), np.nan_to_num(b, nan=-7.0))


def test_noalloc_decode_matches_the_workspace_entry_point():
    print("case: allocation-free decode, B=32 fp8 workload then a B=5 bf16 step", flush=True)
    assert pv.noalloc_scratch_bytes() == 128 << 20
    dec = synth.make("decode_mtp_b32")
    d = to_device(dec)
    for mode in ("refine", "reuse", "dense"):
        ref, ref_s, out, sc = _both(d, 32, 2, 2048, 4096, mode)
        assert np.array_equal(out, ref), mode
        assert _same(sc, ref_s), mode
    del d
    # a second, smaller input in the same scratch array
    small = _small_integer_decode(5, [2, 37, 1000, 999, 1500], 2, 8, 64, 1500, seed=3)
    ds = to_device(small)
    for mode in ("dense", "reuse", "refine"):
        ref, ref_s, out, sc = _both(ds, 5, 2, 40, 100, mode)
        assert np.array_equal(out, ref), mode
        assert _same(sc, ref_s), mode
        for b in range(5):  # and the oracle, exactly (integer inputs)
            r, _, _ = oracle.decode_seq(small, b, 40, 100, mode)
            assert np.array_equal(out[b], r), (mode, b)


def test_noalloc_refuses_a_step_beyond_its_scratch():
    """A dense step over 64 sequences of up to 262144 keys needs more than the
    128 MiB array (its score rows alone take 128 MiB): refused on the host,
    nothing launched, out untouched."""
    print("case: allocation-free decode refuses an oversized step", flush=True)
    B, g, H, D, Lmax = 64, 2, 8, 64, 1 << 18
    assert pv.decode_workspace_size(B, Lmax, H, D, g, 64, 128, "dense", 0) > pv.noalloc_scratch_bytes()
    q = torch.zeros((B, g, H, D), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((B, g, H), dtype=torch.float32, device="cuda")
    k = torch.empty((B, Lmax, D), dtype=torch.bfloat16, device="cuda")
    cl = torch.full((B,), 10, dtype=torch.int32, device="cuda")
    out = torch.full((B, g, 64), 5, dtype=torch.int32, device="cuda")
    with pytest.raises(pv.PivotError, match="scratch"):
        pv.indexer_decode_noalloc(q, w, k, cl, topk=64, C=128, mode="dense", out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 5)  # nothing ran
