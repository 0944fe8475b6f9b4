"""Pins of the oracle's cross-layer index reuse (IndexCache stacked on PIVOT;
molayo1419.me "PIVOT explained", Try it now and Sources -- only the title is
on the pages, so the reading is: full layers run their own indexer, every
other layer takes the rows of the nearest full layer before it).  Checked
against facts that do not come from the reuse code itself: the identity
with per-layer indexing when every layer is full, the identity across
patterns when every layer has the same inputs, and the source layer of each
reusing layer derived by a cumulative maximum over the full layers' indices.
Parity of the reuse with the paper itself is unpinned (the pages give no
algorithm or numbers for it).  CPU only."""
import numpy as np
import pytest

import oracle
import synth

L, H, D, G, K, C = 96, 2, 32, 4, 8, 16


def _layers(n, same=False):
    if same:
        inp = synth.tiny_integer(L=L, H=H, D=D, seed=40)
        return [oracle.View.of(inp)] * n
    return [oracle.View.of(synth.tiny_integer(L=L, H=H, D=D, seed=40 + l)) for l in range(n)]


def _source_by_cummax(full):
    idx = np.where(np.asarray(full, bool), np.arange(len(full)), -1)
    return np.maximum.accumulate(idx)


@pytest.mark.parametrize("mode", ["dense", "reuse", "refine"])
def test_every_layer_full_is_per_layer_indexing(mode):
    views = _layers(4)
    groups = np.arange(L // G)
    got = oracle.index_cache_prefill(views, L, G, K, C, mode, [1, 1, 1, 1], groups)
    for l, v in enumerate(views):
        ref, _ = oracle.prefill_groups(v, L, G, K, C, mode, groups)
        assert np.array_equal(got[l], ref)


@pytest.mark.parametrize("full", [[1, 0, 0, 0], [1, 0, 1, 0], [1, 1, 0, 1], [1, 0, 0, 1, 0, 1]])
def test_same_inputs_give_the_same_rows_whatever_the_pattern(full):
    views = _layers(len(full), same=True)
    groups = np.arange(L // G)
    ref, _ = oracle.prefill_groups(views[0], L, G, K, C, "refine", groups)
    for rows in oracle.index_cache_prefill(views, L, G, K, C, "refine", full, groups):
        assert np.array_equal(rows, ref)


@pytest.mark.parametrize("seed", range(5))
def test_reusing_layers_take_the_nearest_full_layer_before_them(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 7))
    full = [1] + [int(x) for x in rng.integers(0, 2, n - 1)]
    views = _layers(n)
    groups = np.arange(L // G)
    got = oracle.index_cache_prefill(views, L, G, K, C, "refine", full, groups)
    src = _source_by_cummax(full)
    for l in range(n):
        ref, _ = oracle.prefill_groups(views[src[l]], L, G, K, C, "refine", groups)
        assert np.array_equal(got[l], ref), (full, l)
        if src[l] != l:  # a reusing layer's own indexer would differ on these inputs
            own, _ = oracle.prefill_groups(views[l], L, G, K, C, "refine", groups)
            assert not np.array_equal(own, ref)


def test_layer_zero_must_run_its_indexer():
    with pytest.raises(ValueError):
        oracle.index_cache_prefill(_layers(2), L, G, K, C, "refine", [0, 1], np.arange(2))


def test_decode_layers_follow_the_same_rule():
    decs = [synth.decode_mtp(B=3, Lmin=40, Lmax=90, H=2, D=64, g=2, seed=70 + l) for l in range(3)]
    lens = decs[0].cache_len
    for d in decs:
        d.cache_len[:] = lens
    full = [1, 0, 1]
    src = _source_by_cummax(full)
    for b in range(3):
        got = oracle.index_cache_decode(decs, b, 8, 16, "refine", full)
        for l in range(3):
            ref, _, _ = oracle.decode_seq(decs[src[l]], b, 8, 16, "refine")
            assert np.array_equal(got[l], ref)
