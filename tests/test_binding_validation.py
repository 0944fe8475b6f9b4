"""The Python binding rejects tensors that do not match the C ABI's layout
before anything reaches the library: wrong shapes, dtypes or code types,
missing or superfluous fp8 scales, and caller-supplied outputs of the wrong
shape.  CPU only: every case fails on the host (no device, no kernel)."""
import numpy as np
import pytest
import torch

import top_token_selection_pivot_amd as pv


@pytest.fixture(scope="module", autouse=True)
def lib():
    import os
    if not os.path.exists(pv.library_path()):
        from top_token_selection_pivot_amd import build
        build.build(verbose=False)
    return pv.load()


bf, f8, f32, i32 = torch.bfloat16, torch.float8_e4m3fn, torch.float32, torch.int32


def z(shape, dt):
    return torch.zeros(shape, dtype=dt)


def prefill(L=16, H=4, D=32, dt=bf, **over):
    a = dict(q=z((L, H, D), dt), w=z((L, H), f32), k=z((L, D), dt), q_scale=None, k_scale=None)
    if dt == f8:
        a["q_scale"], a["k_scale"] = z((L,), f32), z((L,), f32)
    a.update(over)
    return a


def expect_error(fn, match):
    with pytest.raises(pv.PivotError, match=match):
        fn()


@pytest.mark.parametrize("over,match", [
    (dict(q=z((16, 4, 32), torch.float16)), "code type"),          # 2-byte but not bf16
    (dict(q=z((16, 4, 32), torch.uint8)), "code type"),            # 1-byte but not e4m3
    (dict(q=z((16, 4, 32), torch.float8_e5m2)), "code type"),
    (dict(q=z((16, 4), bf)), r"\[L, H, D\]"),
    (dict(w=z((16, 5), f32)), "w must have shape"),
    (dict(w=z((16, 4), torch.float64)), "w must be"),
    (dict(k=z((15, 32), bf)), "k must have shape"),
    (dict(k=z((16, 64), bf)), "k must have shape"),
    (dict(k=z((16, 32), f8)), "k must be"),
    (dict(q_scale=z((16,), f32)), "take no q_scale"),
])
def test_prefill_rejections(over, match):
    a = prefill(**over)
    expect_error(lambda: pv.indexer(a["q"], a["w"], a["k"], g=4, topk=4, C=8,
                                    q_scale=a["q_scale"], k_scale=a["k_scale"]), match)


def test_fp8_scales_required_and_shaped():
    a = prefill(D=64, dt=f8)
    expect_error(lambda: pv.indexer(a["q"], a["w"], a["k"], g=4, topk=4, C=8, q_scale=None,
                                    k_scale=a["k_scale"]), "q_scale is required")
    expect_error(lambda: pv.indexer(a["q"], a["w"], a["k"], g=4, topk=4, C=8, q_scale=z((15,), f32),
                                    k_scale=a["k_scale"]), "q_scale must have shape")
    expect_error(lambda: pv.indexer(a["q"], a["w"], a["k"], g=4, topk=4, C=8, q_scale=a["q_scale"],
                                    k_scale=z((16,), torch.float64)), "k_scale must be")


def test_outputs_are_checked():
    a = prefill()
    run = lambda **kw: pv.indexer(a["q"], a["w"], a["k"], g=4, topk=4, C=8, **kw)
    expect_error(lambda: run(out=z((16, 5), i32)), "out must have shape")
    expect_error(lambda: run(out=z((16, 4), torch.int64)), "out must be")
    # with a window the rows are topk + window wide
    expect_error(lambda: run(out=z((16, 4), i32), window=3), "out must have shape")
    expect_error(lambda: run(out_scores=z((16, 4), torch.float64)), "out_scores must be")
    expect_error(lambda: run(return_scores=True, window=2), "without a window")
    expect_error(lambda: run(mode="sparse"), "mode")
    expect_error(lambda: run(window_mode=5, window=2), "window_mode")


def test_cpu_tensors_are_refused_after_the_shape_checks():
    a = prefill()
    expect_error(lambda: pv.indexer(a["q"], a["w"], a["k"], g=4, topk=4, C=8), "device tensor")


def decode(B=3, g=2, H=4, D=64, Lmax=100, dt=f8, **over):
    a = dict(q=z((B, g, H, D), dt), w=z((B, g, H), f32), k=z((B, Lmax, D), dt),
             cl=z((B,), i32), qs=z((B, g), f32), ks=z((B, Lmax), f32))
    a.update(over)
    return a


@pytest.mark.parametrize("over,match", [
    (dict(q=z((3, 2, 4), f8)), r"\[B, g, H, D\]"),
    (dict(w=z((3, 2, 5), f32)), "w must have shape"),
    (dict(k=z((2, 100, 64), f8)), "k_cache must have shape"),
    (dict(k=z((3, 100, 32), f8)), "k_cache must have shape"),
    (dict(cl=z((4,), i32)), "cache_len must have shape"),
    (dict(cl=z((3,), torch.int64)), "cache_len must be"),
    (dict(qs=z((3, 1), f32)), "q_scale must have shape"),
    (dict(ks=z((3, 99), f32)), "k_scale must have shape"),
])
def test_decode_rejections(over, match):
    a = decode(**over)
    expect_error(lambda: pv.indexer_decode(a["q"], a["w"], a["k"], a["cl"], topk=8, C=16,
                                           q_scale=a["qs"], k_scale=a["ks"]), match)
    if "k" not in over and "cl" not in over:
        expect_error(lambda: pv.decode_candidates(a["q"], a["w"], a["k"], a["cl"], topk=8, C=16,
                                                  q_scale=a["qs"], k_scale=a["ks"]), match)


def test_decode_outputs_are_checked():
    a = decode()
    run = lambda **kw: pv.indexer_decode(a["q"], a["w"], a["k"], a["cl"], topk=8, C=16,
                                         q_scale=a["qs"], k_scale=a["ks"], **kw)
    expect_error(lambda: run(out=z((3, 2, 9), i32)), "out must have shape")
    expect_error(lambda: run(out=z((3, 2, 8), i32), window=4), "out must have shape")
    expect_error(lambda: run(out_scores=z((3, 2, 7), f32)), "out_scores must have shape")


def test_paged_rejections():
    a = decode()
    kp, ksp, bt = z((10, 64, 64), f8), z((10, 64), f32), z((3, 2), i32)
    run = lambda **kw: pv.indexer_decode_paged(
        kw.get("q", a["q"]), a["w"], kw.get("kp", kp), kw.get("bt", bt), a["cl"], topk=8, C=16,
        q_scale=a["qs"], k_scale=kw.get("ksp", ksp))
    expect_error(lambda: run(kp=z((10, 64, 32), f8)), "k_pages must have shape")
    expect_error(lambda: run(ksp=z((10, 32), f32)), "k_scale must have shape")
    expect_error(lambda: run(bt=z((2, 2), i32)), "block_table must have shape")
    expect_error(lambda: run(bt=z((3, 2), torch.int64)), "block_table must be")
    expect_error(lambda: run(kp=z((10, 64, 64), bf)), "k_pages must be")


def test_varlen_rejections():
    a = prefill(L=20)
    run = lambda cu: pv.indexer_varlen(a["q"], a["w"], a["k"], cu, g=4, topk=4, C=8)
    expect_error(lambda: run([0, 10, 19]), "cu_seqlens")
    expect_error(lambda: run([1, 20]), "cu_seqlens")
    expect_error(lambda: run([20]), "cu_seqlens")


def test_proxy_mean_and_score_rows_rejections():
    a = prefill()
    expect_error(lambda: pv.proxy_mean(a["q"], z((16, 3), f32), 4), "w must have shape")
    expect_error(lambda: pv.proxy_mean(z((16, 4, 64), f8), a["w"], 4), "q_scale is required")
    expect_error(lambda: pv.score_rows(a["q"], a["w"], z((40, 64), bf)), "k must have shape")
    expect_error(lambda: pv.score_rows(a["q"], a["w"], z((40,), bf)), r"\[Lk, D\]")


def test_sparse_attention_rejections():
    q, k, v, idx = z((8, 32, 128), bf), z((100, 128), bf), z((100, 128), bf), z((8, 16), i32)
    expect_error(lambda: pv.sparse_attention(z((8, 32, 128), torch.float16), k, v, idx), "bf16")
    expect_error(lambda: pv.sparse_attention(q, z((100, 64), bf), v, idx), "k must have shape")
    expect_error(lambda: pv.sparse_attention(q, k, z((99, 128), bf), idx), "v must have shape")
    expect_error(lambda: pv.sparse_attention(q, k, v, z((7, 16), i32)), "idx must have shape")
    expect_error(lambda: pv.sparse_attention(q, k, v, z((8, 16), torch.int64)), "idx must be")
    expect_error(lambda: pv.sparse_attention(q, k, v, idx, seq_len=101), "seq_len")
    expect_error(lambda: pv.sparse_attention(q, k, v, idx, out=z((8, 32, 64), f32)), "out must have shape")
    kb = z((2, 50, 128), bf)
    expect_error(lambda: pv.sparse_attention(q, kb, kb, idx, rows_per_seq=2), "sequences")
