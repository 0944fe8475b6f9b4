"""GPU parity of cross-layer index reuse stacked on the indexer
(pivot_indexer_layers / pivot_indexer_decode_layers): full layers run the
indexer on their own inputs, the other layers take the rows of the nearest
full layer before them.  Integer-valued inputs: bit-exact against the
oracle in every mode; the reuse itself is exact at any size (a copy), checked
on the 16K float workload against single-layer calls."""
import numpy as np
import pytest
import torch

import oracle
import synth
import top_token_selection_pivot_amd as pv
from parity import to_device

pytestmark = pytest.mark.gpu

L, H, D, G, K, C = 2048, 4, 32, 4, 64, 256


@pytest.fixture(scope="module")
def layers():
    inps = [synth.tiny_integer(L=L, H=H, D=D, seed=2000 + l) for l in range(4)]
    return inps, [to_device(x) for x in inps]


@pytest.mark.parametrize("mode", ["dense", "reuse", "refine"])
@pytest.mark.parametrize("full", [[1, 1, 1, 1], [1, 0, 1, 0], [1, 0, 0, 0], [1, 1, 0, 1]])
def test_prefill_layers_bit_exact(layers, mode, full):
    print(f"case: {len(full)} layers {full}, tiny prefill, {mode}", flush=True)
    inps, ds = layers
    qs = [d["q"] if f else None for d, f in zip(ds, full)]
    ws = [d["w"] if f else None for d, f in zip(ds, full)]
    ks = [d["k"] if f else None for d, f in zip(ds, full)]
    outs = pv.indexer_layers(qs, ws, ks, full=full, g=G, topk=K, C=C, mode=mode)
    torch.cuda.synchronize()
    ref = oracle.index_cache_prefill([oracle.View.of(x) for x in inps], L, G, K, C, mode, full,
                                     np.arange(L // G))
    for l in range(len(full)):
        assert np.array_equal(outs[l].cpu().numpy(), ref[l]), l


def test_aliased_outputs_are_left_to_the_source(layers):
    print("case: layers with the reusing layer's output aliased to its source", flush=True)
    inps, ds = layers
    out0 = torch.full((L, K), -7, dtype=torch.int32, device="cuda")
    out2 = torch.full((L, K), -7, dtype=torch.int32, device="cuda")
    full = [1, 0, 1]
    outs = pv.indexer_layers([ds[0]["q"], None, ds[2]["q"]], [ds[0]["w"], None, ds[2]["w"]],
                             [ds[0]["k"], None, ds[2]["k"]], full=full, g=G, topk=K, C=C,
                             mode="refine", outs=[out0, out0, out2])
    torch.cuda.synchronize()
    ref = oracle.index_cache_prefill([oracle.View.of(x) for x in inps[:3]], L, G, K, C, "refine", full,
                                     np.arange(L // G))
    assert outs[1] is out0
    assert np.array_equal(out0.cpu().numpy(), ref[0]) and np.array_equal(out2.cpu().numpy(), ref[2])


def _small_decode(seed, lens, dtype):
    rng = np.random.default_rng(seed)
    B, g, Hd, Dd, Lmax = len(lens), 2, 8, 64, max(lens)
    qf = rng.integers(-2, 3, (B, g, Hd, Dd)).astype(np.float32)
    kf = rng.integers(-2, 3, (B, Lmax, Dd)).astype(np.float32)
    w = rng.integers(1, 4, (B, g, Hd)).astype(np.float32)
    if dtype == "bf16":
        return synth.DecodeInputs("bf16", B, Lmax, Hd, Dd, g, synth.encode_bf16(qf), None, w,
                                  synth.encode_bf16(kf), None, np.asarray(lens, np.int32))
    return synth.DecodeInputs("fp8", B, Lmax, Hd, Dd, g, synth._encode_fp8(qf), np.ones((B, g), np.float32),
                              w, synth._encode_fp8(kf), np.ones((B, Lmax), np.float32),
                              np.asarray(lens, np.int32))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_decode_layers_bit_exact(dtype):
    print(f"case: 3 decode layers [1, 0, 1], {dtype}", flush=True)
    lens = [2, 40, 777, 1500, 1200]
    decs = [_small_decode(500 + l, lens, dtype) for l in range(3)]
    ds = [to_device(x) for x in decs]
    full = [1, 0, 1]
    for mode in ("dense", "reuse", "refine"):
        outs = pv.indexer_decode_layers([d["q"] for d in ds], [d["w"] for d in ds], [d["k"] for d in ds],
                                        ds[0]["cache_len"], full=full, topk=40, C=100, mode=mode,
                                        q_scales=[d["q_scale"] for d in ds], k_scales=[d["k_scale"] for d in ds])
        torch.cuda.synchronize()
        for b in range(len(lens)):
            ref = oracle.index_cache_decode(decs, b, 40, 100, mode, full)
            for l in range(3):
                assert np.array_equal(outs[l][b].cpu().numpy(), ref[l]), (mode, b, l)


def test_reuse_is_exact_on_the_16k_workload():
    print("case: 2 layers [1, 0] on the 16K bf16 workload, Refine g=8", flush=True)
    inp = synth.make("dsa_prefill_16k")
    d = to_device(inp)
    outs = pv.indexer_layers([d["q"], None], [d["w"], None], [d["k"], None], full=[1, 0], g=8, topk=2048,
                             C=4096, mode="refine")
    single = pv.indexer(d["q"], d["w"], d["k"], g=8, topk=2048, C=4096, mode="refine")
    torch.cuda.synchronize()
    assert torch.equal(outs[0], single) and torch.equal(outs[1], single)
