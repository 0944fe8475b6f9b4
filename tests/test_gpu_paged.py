"""GPU parity of the decode step over a paged indexer-key cache
(pivot_indexer_decode_paged).  The keys of every sequence sit in shuffled
pages of a shared pool whose other bytes are random codes; the expected rows
are the oracle's decode step over the contiguous cache the block table stands
for (oracle.paged_keys).  Integer-valued inputs, so rows must match bit for
bit; at the full B=32, 128K-key fp8 decode workload the paged call must also
equal the contiguous call row for row (paging changes addresses only)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
import top_token_selection_pivot_amd as pv
from parity import EPS_FP8, check_band, to_device

pytestmark = pytest.mark.gpu


def _decode_inputs(B, lens, g, H=8, D=64, dtype="bf16", Lmax=None, seed=3):
    Lmax = Lmax or max(lens)
    rng = np.random.default_rng(seed)
    qf = rng.integers(-2, 3, (B, g, H, D)).astype(np.float32)
    kf = rng.integers(-2, 3, (B, Lmax, D)).astype(np.float32)
    w = rng.integers(1, 4, (B, g, H)).astype(np.float32)
    if dtype == "bf16":
        return synth.DecodeInputs("bf16", B, Lmax, H, D, g, synth.encode_bf16(qf), None, w,
                                  synth.encode_bf16(kf), None, np.asarray(lens, np.int32))
    return synth.DecodeInputs("fp8", B, Lmax, H, D, g, synth._encode_fp8(qf),
                              np.ones((B, g), np.float32), w, synth._encode_fp8(kf),
                              np.ones((B, Lmax), np.float32), np.asarray(lens, np.int32))


def _pages_dev(pc):
    if pc.k_pages.dtype == np.uint16:
        kp = torch.from_numpy(pc.k_pages.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        kp = torch.from_numpy(pc.k_pages).view(torch.float8_e4m3fn).cuda()
    ks = None if pc.k_scale_pages is None else torch.from_numpy(pc.k_scale_pages).cuda()
    return kp, ks, torch.from_numpy(pc.block_table).cuda()


def _run_paged(dec, pc, **kw):
    d = to_device(dec)
    kp, ks, bt = _pages_dev(pc)
    out = pv.indexer_decode_paged(d["q"], d["w"], kp, bt, d["cache_len"], q_scale=d["q_scale"],
                                  k_scale=ks, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _oracle_rows(dec, pc, topk, C, mode, W=0, wmode="shared"):
    k, ks = oracle.paged_keys(pc.k_pages, pc.k_scale_pages, pc.block_table, dec.cache_len, dec.Lmax)
    view = dataclasses.replace(dec, k=k, k_scale=ks)
    rows = []
    for b in range(dec.B):
        if W:
            rows.append(oracle.decode_seq_window(view, b, topk, C, mode, W, wmode)[0])
        else:
            rows.append(oracle.decode_seq(view, b, topk, C, mode)[0])
    return np.stack(rows)


LENS = [2, 63, 64, 65, 1000, 1500, 777]


@pytest.mark.parametrize("page_size", [64, 256])
@pytest.mark.parametrize("mode", ["dense", "reuse", "refine"])
def test_paged_decode_exact(mode, page_size):
    print(f"case: paged decode bf16 B=7 page {page_size} {mode}", flush=True)
    dec = _decode_inputs(7, LENS, g=2, H=8, D=64, Lmax=1500, seed=page_size)
    pc = synth.paged_cache(dec, page_size, seed=11)
    out = _run_paged(dec, pc, topk=40, C=100, mode=mode)
    assert np.array_equal(out, _oracle_rows(dec, pc, 40, 100, mode))
    d = to_device(dec)
    flat = pv.indexer_decode(d["q"], d["w"], d["k"], d["cache_len"], topk=40, C=100, mode=mode)
    assert np.array_equal(out, flat.cpu().numpy())


@pytest.mark.parametrize("mode", ["dense", "refine"])
def test_paged_decode_fp8_many_sequences(mode):
    # about 1100 key pairs: the decode scan's runs of pairs start and end
    # inside sequences and pages
    print(f"case: paged decode fp8 B=24 H=64 D=128 page 64 {mode}", flush=True)
    rng = np.random.default_rng(21)
    lens = [int(x) for x in rng.integers(2, 6000, 24)]
    lens[3], lens[7], lens[8], lens[9] = 6000, 64, 65, 2
    dec = _decode_inputs(24, lens, g=2, H=64, D=128, dtype="fp8", Lmax=6000, seed=22)
    pc = synth.paged_cache(dec, 64, seed=12)
    out = _run_paged(dec, pc, topk=64, C=256, mode=mode)
    assert np.array_equal(out, _oracle_rows(dec, pc, 64, 256, mode))


@pytest.mark.parametrize("g,mode", [(4, "dense"), (4, "refine"), (3, "reuse")])
def test_paged_decode_deeper_mtp(g, mode):
    print(f"case: paged decode bf16 B=5 g={g} page 128 {mode}", flush=True)
    lens = [g, 130, 128, 700, 1023]
    dec = _decode_inputs(5, lens, g=g, H=16, D=128, Lmax=1100, seed=g)
    pc = synth.paged_cache(dec, 128, seed=13)
    out = _run_paged(dec, pc, topk=48, C=160, mode=mode)
    assert np.array_equal(out, _oracle_rows(dec, pc, 48, 160, mode))


@pytest.mark.parametrize("wmode", ["shared", "excluded"])
@pytest.mark.parametrize("mode", ["dense", "refine"])
def test_paged_decode_window(mode, wmode):
    print(f"case: paged decode bf16 B=7 page 128 window 64 {wmode} {mode}", flush=True)
    dec = _decode_inputs(7, LENS, g=2, H=8, D=64, Lmax=1500, seed=7)
    pc = synth.paged_cache(dec, 128, seed=14)
    out = _run_paged(dec, pc, topk=40, C=100, mode=mode, window=64, window_mode=wmode)
    assert np.array_equal(out, _oracle_rows(dec, pc, 40, 100, mode, 64, wmode))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_paged_decode_page_ids_outside_pool(dtype):
    # an id outside the pool reads as a page of zero keys (scores 0)
    print(f"case: paged decode {dtype} with page ids outside the pool", flush=True)
    D = 64 if dtype == "bf16" else 128
    dec = _decode_inputs(7, LENS, g=2, H=8, D=D, dtype=dtype, Lmax=1500, seed=9)
    pc = synth.paged_cache(dec, 64, seed=15)
    npages = pc.k_pages.shape[0]
    pc.block_table[4, 3] = npages + 3
    pc.block_table[5, 0] = -5
    pc.block_table[6, 12] = 1 << 30
    for mode in ("dense", "refine"):
        out = _run_paged(dec, pc, topk=40, C=100, mode=mode)
        assert np.array_equal(out, _oracle_rows(dec, pc, 40, 100, mode)), mode


def test_paged_decode_mtp_b32():
    print("case: paged decode B=32 g=2 fp8 k=2048 C=4096 page 64, cache lengths in [32768, 131072]",
          flush=True)
    dec = synth.make("decode_mtp_b32")
    pc = synth.paged_cache(dec, 64, seed=16)
    d = to_device(dec)
    kp, ks, bt = _pages_dev(pc)
    for mode in ("refine", "reuse", "dense"):
        kw = dict(topk=2048, C=4096, mode=mode, q_scale=d["q_scale"])
        paged = pv.indexer_decode_paged(d["q"], d["w"], kp, bt, d["cache_len"], k_scale=ks, **kw)
        flat = pv.indexer_decode(d["q"], d["w"], d["k"], d["cache_len"], k_scale=d["k_scale"], **kw)
        assert torch.equal(paged, flat), mode
        print(f"paged == contiguous, {mode}: ok", flush=True)
    # the oracle reads two sequences through the block table
    out = paged.cpu().numpy()  # dense rows
    for b in (0, 31):
        sub = pc.block_table[b:b + 1]
        k, kss = oracle.paged_keys(pc.k_pages, pc.k_scale_pages, sub, dec.cache_len[b:b + 1], dec.Lmax)
        v = oracle.View(dec.dtype, dec.q[b], dec.q_scale[b], dec.w[b], k[0], kss[0])
        n = int(dec.cache_len[b])
        for i in range(2):
            t = n - 2 + i
            sc = oracle.score_row(v, i, t + 1)
            check_band(out[b, i], np.arange(t + 1), sc, 2048, EPS_FP8, f"paged dense seq {b}")
    print("paged dense rows against the oracle: ok", flush=True)
