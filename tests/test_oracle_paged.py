"""CPU pins of the oracle's paged-cache view (oracle.paged_keys): a hand-worked
block table, and the round trip through the seeded page layout that the GPU
tests use (scatter a contiguous cache into shuffled pages, read it back)."""
import numpy as np

import oracle
import synth


def test_paged_keys_hand_example():
    # pool of 3 pages of 2 one-element keys; sequence 0 uses pages 2, 0 and
    # holds 3 keys, sequence 1 uses page 1 and an id outside the pool
    pages = np.array([[[10], [11]], [[20], [21]], [[30], [31]]], np.uint16)
    scales = np.array([[1.0, 1.5], [2.0, 2.5], [3.0, 3.5]], np.float32)
    bt = np.array([[2, 0], [1, 7]], np.int32)
    k, ks = oracle.paged_keys(pages, scales, bt, np.array([3, 4], np.int32), 4)
    assert k[:, :, 0].tolist() == [[30, 31, 10, 0], [20, 21, 0, 0]]
    assert ks.tolist() == [[3.0, 3.5, 1.0, 0.0], [2.0, 2.5, 0.0, 0.0]]
    k, ks = oracle.paged_keys(pages, None, bt[:1], np.array([2], np.int32), 4)
    assert ks is None and k[0, :, 0].tolist() == [30, 31, 0, 0]


def _dec(dtype, lens, Lmax, D=32):
    rng = np.random.default_rng(5)
    B = len(lens)
    kf = rng.integers(-3, 4, (B, Lmax, D)).astype(np.float32)
    qf = rng.integers(-3, 4, (B, 2, 2, D)).astype(np.float32)
    w = np.ones((B, 2, 2), np.float32)
    if dtype == "bf16":
        return synth.DecodeInputs("bf16", B, Lmax, 2, D, 2, synth.encode_bf16(qf), None, w,
                                  synth.encode_bf16(kf), None, np.asarray(lens, np.int32))
    kc, ks = synth.encode_fp8_per_row(kf, 2)
    qc, qs = synth.encode_fp8_per_row(qf, 2)
    return synth.DecodeInputs("fp8", B, Lmax, 2, D, 2, qc, qs, w, kc, ks, np.asarray(lens, np.int32))


def test_paged_layout_round_trip():
    for dtype in ("bf16", "fp8"):
        for ps in (64, 128):
            lens = [2, 64, 65, 300, 1]
            dec = _dec(dtype, lens, 300)
            pc = synth.paged_cache(dec, ps, seed=ps)
            # every page is used once, the spare ones by nobody
            ids = pc.block_table[pc.block_table >= 0]
            assert len(set(ids.tolist())) == ids.size == sum((n + ps - 1) // ps for n in lens)
            k, ks = oracle.paged_keys(pc.k_pages, pc.k_scale_pages, pc.block_table, dec.cache_len,
                                      dec.Lmax)
            for b, n in enumerate(lens):
                assert np.array_equal(k[b, :n], dec.k[b, :n]), (dtype, ps, b)
                assert not k[b, n:].any()
                if dtype == "fp8":
                    assert np.array_equal(ks[b, :n], dec.k_scale[b, :n])
