"""GPU parity of several prefill sequences in one call (variable lengths, one
after another in the inputs): every sequence's rows must equal the oracle's for
that sequence alone (integer-valued inputs: bit for bit), in every mode, with
and without a sliding window, for bf16 and fp8 codes (per-token scales), including
empty and one-token sequences."""
import numpy as np
import pytest
import torch

import oracle
import synth
import top_token_selection_pivot_amd as pv
from parity import to_device

pytestmark = pytest.mark.gpu

LENS = [37, 0, 1, 700, 2048, 5, 300]


@pytest.fixture(scope="module")
def batch():
    inp = synth.small_integer(sum(LENS), 4, 32, seed=77, qmax=2, kmax=2, wmax=3)
    cu = np.concatenate([[0], np.cumsum(LENS)]).astype(np.int64)
    return inp, cu


def _seq_view(inp, a, b):
    return oracle.View("bf16", inp.q[a:b], None, inp.w[a:b], inp.k[a:b], None)


@pytest.mark.parametrize("W,wmode", [(0, "shared"), (16, "shared"), (16, "excluded")])
@pytest.mark.parametrize("mode", ["dense", "reuse", "refine"])
def test_varlen_bit_exact(batch, mode, W, wmode):
    print(f"case: varlen prefill lengths {LENS} g=4 k=24 C=60 {mode} window {W} {wmode}", flush=True)
    inp, cu = batch
    d = to_device(inp)
    got = pv.indexer_varlen(d["q"], d["w"], d["k"], cu, g=4, topk=24, C=60, mode=mode, window=W,
                            window_mode=wmode).cpu().numpy()
    assert got.shape == (cu[-1], 24 + W)
    for i, L in enumerate(LENS):
        if L == 0:
            continue
        a, b = int(cu[i]), int(cu[i + 1])
        v = _seq_view(inp, a, b)
        excl = W if wmode == "excluded" else 0
        if mode == "dense":
            sel = oracle.dense_rows(v, np.arange(L), 24, excl=excl)
        else:
            sel, _ = oracle.prefill_groups(v, L, 4, 24, 60, mode, np.arange((L + 3) // 4), excl=excl)
        ref = oracle.window_union(sel, np.arange(L), W) if W else sel
        assert np.array_equal(got[a:b], ref), (mode, i)


def test_varlen_equals_separate_calls(batch):
    print("case: varlen == one call per sequence (Refine g=4)", flush=True)
    inp, cu = batch
    d = to_device(inp)
    got = pv.indexer_varlen(d["q"], d["w"], d["k"], cu, g=4, topk=24, C=60, mode="refine")
    for i, L in enumerate(LENS):
        if L == 0:
            continue
        a, b = int(cu[i]), int(cu[i + 1])
        one = pv.indexer(d["q"][a:b].contiguous(), d["w"][a:b].contiguous(), d["k"][a:b].contiguous(),
                         g=4, topk=24, C=60, mode="refine")
        assert torch.equal(got[a:b], one), i


LENS8 = [129, 0, 1, 1000, 3, 260]


@pytest.mark.parametrize("mode", ["dense", "reuse", "refine"])
def test_varlen_fp8_bit_exact(mode):
    # fp8 codes of small integers with unit scales: every sum is exact, so the
    # packed call must reproduce each sequence's oracle rows bit for bit
    print(f"case: varlen fp8 prefill lengths {LENS8} g=8 k=32 C=96 {mode}", flush=True)
    inp = synth.small_integer(sum(LENS8), 8, 64, seed=91, qmax=2, kmax=2, wmax=3, dtype="fp8")
    cu = np.concatenate([[0], np.cumsum(LENS8)]).astype(np.int64)
    d = to_device(inp)
    got = pv.indexer_varlen(d["q"], d["w"], d["k"], cu, g=8, topk=32, C=96, mode=mode,
                            q_scale=d["q_scale"], k_scale=d["k_scale"]).cpu().numpy()
    assert got.shape == (cu[-1], 32)
    for i, L in enumerate(LENS8):
        if L == 0:
            continue
        a, b = int(cu[i]), int(cu[i + 1])
        v = oracle.View("fp8", inp.q[a:b], inp.q_scale[a:b], inp.w[a:b], inp.k[a:b], inp.k_scale[a:b])
        if mode == "dense":
            ref = oracle.dense_rows(v, np.arange(L), 32)
        else:
            ref, _ = oracle.prefill_groups(v, L, 8, 32, 96, mode, np.arange((L + 7) // 8))
        assert np.array_equal(got[a:b], ref), (mode, i)


def test_varlen_rows_do_not_depend_on_the_workspace(batch):
    """The preferred workspace runs sequences concurrently on the library's
    streams; the longest sequence's minimum runs them one after another on the
    caller's stream; both (and two slices) give identical rows."""
    print("case: varlen with the preferred, a two-slice and the minimum workspace", flush=True)
    inp, cu = batch
    d = to_device(inp)
    kw = dict(g=4, topk=24, C=60, mode="refine")
    ref = pv.indexer_varlen(d["q"], d["w"], d["k"], cu, **kw)
    L = pv.load()
    lmax = int(np.max(np.diff(cu)))
    mn = L.pivot_workspace_min_size(lmax, 4, 32, 4, 24, 60, pv.REFINE, 0)
    pref = L.pivot_workspace_size(lmax, 4, 32, 4, 24, 60, pv.REFINE, 0)
    for nbytes in (mn, 2 * ((pref + 255) // 256 * 256)):
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        got = pv.indexer_varlen(d["q"], d["w"], d["k"], cu, workspace=ws, **kw)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), nbytes
