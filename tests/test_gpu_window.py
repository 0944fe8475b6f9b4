"""GPU parity of the sliding window added to the selection (tutorial "Sparse
Attention의 Indexer", section on combining the recent window with the selected
positions, Figure 3), both designs: the window's positions stay candidates
(union with the selection) or are excluded (each query chooses among 0..t-W).
Integer-valued inputs, so every row must match the oracle bit for bit."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
import top_token_selection_pivot_amd as pv
from conftest import GOLDEN
from parity import to_device

pytestmark = pytest.mark.gpu


def _run(inp, mode, g, topk, C, W, wmode, **kw):
    d = to_device(inp)
    out = pv.indexer(d["q"], d["w"], d["k"], g=g, topk=topk, C=C, mode=mode,
                     q_scale=d["q_scale"], k_scale=d["k_scale"], window=W, window_mode=wmode, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _oracle(inp, mode, g, topk, C, W, wmode):
    v = oracle.View.of(inp)
    excl = W if wmode == "excluded" else 0
    if mode == "dense":
        sel = oracle.dense_rows(v, np.arange(inp.L), topk, excl=excl)
    else:
        G = (inp.L + g - 1) // g
        sel, _ = oracle.prefill_groups(v, inp.L, g, topk, C, mode, np.arange(G), excl=excl)
    return oracle.window_union(sel, np.arange(inp.L), W)


def test_window_printed_example():
    print("case: window 3 at p7 (Figure 3) and the excluded-window design", flush=True)
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_fig1.json")))
    wx = json.load(open(os.path.join(GOLDEN, "window_example_fig3.json")))
    a = ex["keys_first_component"]
    b = ex["keys_second_component_p0_to_p6"] + [ex["key_p7_second_component"]]
    q = np.zeros((8, 1, 32), np.float32)
    q[:, 0, 0] = 1
    q[6, 0, :2] = ex["query_p6"]
    q[7, 0, :2] = ex["query_p7"]
    k = np.zeros((8, 32), np.float32)
    k[:, 0], k[:, 1] = a, b
    inp = synth.PrefillInputs("bf16", 8, 1, 32, synth.encode_bf16(q), None, np.ones((8, 1), np.float32),
                              synth.encode_bf16(k), None)
    W = wx["window"]
    out = _run(inp, "dense", 1, 3, 3, W, "shared")
    assert [p for p in out[7].tolist() if p >= 0] == wx["union_p7_printed"]
    assert [p for p in out[6].tolist() if p >= 0] == wx["union_p6_derived"]
    out = _run(inp, "dense", 1, 3, 3, W, "excluded")
    assert out[7].tolist() == wx["excluded_p7_derived"]
    assert out[6].tolist() == wx["excluded_p6_derived"]


@pytest.fixture(scope="module")
def tiny():
    return synth.make("tiny_prefill_2k")


@pytest.mark.parametrize("W", [3, 300])
@pytest.mark.parametrize("wmode", ["shared", "excluded"])
@pytest.mark.parametrize("mode", ["dense", "reuse", "refine"])
def test_window_tiny_prefill_bit_exact(tiny, mode, wmode, W):
    print(f"case: tiny prefill L=2048 g=4 k=64 C=256 {mode} window {W} {wmode}", flush=True)
    got = _run(tiny, mode, 4, 64, 256, W, wmode)
    ref = _oracle(tiny, mode, 4, 64, 256, W, wmode)
    assert got.shape == ref.shape == (2048, 64 + W)
    bad = np.nonzero((got != ref).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} rows differ, first {bad[:5]}"


@pytest.mark.parametrize("wmode", ["shared", "excluded"])
def test_window_chunked_passes_and_long_window(wmode):
    # a workspace for two row blocks forces many passes; a window longer than
    # most prefixes and groups whose whole range lies inside the window
    print(f"case: L=700 H=8 D=64 g=3 k=40 C=90, minimum workspace, windows 1/65/900 {wmode}", flush=True)
    inp = synth.small_integer(700, 8, 64, seed=55, qmax=2, kmax=2, wmax=3)
    for W in (1, 65, 900):
        for mode in ("reuse", "refine", "dense"):
            nmin = pv.load().pivot_workspace_min_size(700, 8, 64, 3, 40, 90, pv._mode(mode), 0)
            ws = torch.empty(nmin, dtype=torch.uint8, device="cuda")
            got = _run(inp, mode, 3, 40, 90, W, wmode, workspace=ws)
            ref = _oracle(inp, mode, 3, 40, 90, W, wmode)
            assert np.array_equal(got, ref), (mode, W)


@pytest.mark.parametrize("wmode", ["shared", "excluded"])
@pytest.mark.parametrize("mode", ["dense", "reuse", "refine"])
def test_window_fp8_prefill_bit_exact(mode, wmode):
    # fp8 codes of small integers with unit scales (every sum exact)
    print(f"case: fp8 prefill L=900 H=8 D=64 g=8 k=48 C=120 {mode} window 37 {wmode}", flush=True)
    inp = synth.small_integer(900, 8, 64, seed=63, qmax=2, kmax=2, wmax=3, dtype="fp8")
    got = _run(inp, mode, 8, 48, 120, 37, wmode)
    ref = _oracle(inp, mode, 8, 48, 120, 37, wmode)
    assert got.shape == ref.shape == (900, 48 + 37)
    bad = np.nonzero((got != ref).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} rows differ, first {bad[:5]}"


def test_window_zero_equals_plain(tiny):
    print("case: window 0 through the window entry point", flush=True)
    d = to_device(tiny)
    L = pv.load()
    for mode in ("dense", "reuse", "refine"):
        m = pv._mode(mode)
        ws = torch.empty(L.pivot_workspace_size(2048, 4, 32, 4, 64, 256, m, 0), dtype=torch.uint8,
                         device="cuda")
        out = torch.full((2048, 64), -7, dtype=torch.int32, device="cuda")
        for wmode in (0, 1):
            pv._check(L.pivot_indexer_window(
                pv._ptr(d["q"]), None, pv._ptr(d["w"]), pv._ptr(d["k"]), None, 2048, 4, 32, 4, 64,
                256, m, 0, 0, wmode, pv._ptr(out), pv._ptr(ws), ws.numel(), None))
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy(), _run(tiny, mode, 4, 64, 256, 0, "shared"))


def _decode_inputs(B, lens, g, H, D, dtype, Lmax, seed):
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


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("fp8", 128)])
@pytest.mark.parametrize("wmode", ["shared", "excluded"])
def test_window_decode_bit_exact(dtype, D, wmode):
    print(f"case: decode B=14 H=16 D={D} {dtype} windows 5/2100 {wmode}", flush=True)
    rng = np.random.default_rng(D)
    lens = [int(x) for x in rng.integers(2, 3000, 14)]
    lens[0], lens[3], lens[5], lens[9] = 1, 3000, 4, 2101   # invalid, full, shorter than a window
    dec = _decode_inputs(14, lens, 2, 16, D, dtype, 3000, seed=D + 1)
    d = to_device(dec)
    kw = dict(q_scale=d["q_scale"], k_scale=d["k_scale"]) if dtype == "fp8" else {}
    for W in (5, 2100):
        for mode in ("dense", "reuse", "refine"):
            out = pv.indexer_decode(d["q"], d["w"], d["k"], d["cache_len"], topk=48, C=160,
                                    mode=mode, window=W, window_mode=wmode, **kw).cpu().numpy()
            assert out.shape == (14, 2, 48 + W)
            for b in range(14):
                if lens[b] < 2:
                    assert np.all(out[b] == -1), (mode, W, b)
                    continue
                ref, _ = oracle.decode_seq_window(dec, b, 48, 160, mode, W, wmode)
                assert np.array_equal(out[b], ref), (mode, W, b)
