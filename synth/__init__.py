"""Seeded synthetic inputs for the PIVOT indexer.

This module only draws inputs: it holds none of the indexer's arithmetic and is
shared by the CPU oracle's tests and the GPU path's tests and benchmark, so both
sides see identical bytes.  Values are drawn in float32 with numpy's PCG64 and
then encoded to the storage type with PyTorch's CPU casts (bf16 round to
nearest even; fp8 OCP E4M3FN round to nearest even after clamping to +-448, with
a per-token float32 scale amax/448).

Workload shapes follow the DSA indexer as the pages describe it (several
indexer heads, one indexer key per token shared by every head, long context);
the distributions give correlated neighbouring queries and long-tailed key
norms, the two properties PIVOT relies on (arXiv:2607.24593 abstract).  They
stand in for the LongBench/RULER runs of DeepSeek-V3.2/GLM-5.1, which need
datasets and trained weights that are not used here.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

__all__ = [
    "PrefillInputs",
    "DecodeInputs",
    "encode_bf16",
    "encode_fp8_per_row",
    "tiny_integer",
    "small_integer",
    "dsa_prefill",
    "decode_mtp",
    "PagedCache",
    "paged_cache",
    "CONFIGS",
]


@dataclass
class PrefillInputs:
    """One prefill sequence: L queries and L keys.

    q: [L,H,D] codes (uint16 bf16 or uint8 E4M3FN); q_scale: [L] float32 (fp8 only)
    w: [L,H] float32 head weights
    k: [L,D] codes; k_scale: [L] float32 (fp8 only)
    """

    dtype: str
    L: int
    H: int
    D: int
    q: np.ndarray
    q_scale: Optional[np.ndarray]
    w: np.ndarray
    k: np.ndarray
    k_scale: Optional[np.ndarray]


@dataclass
class DecodeInputs:
    """One multi-token-prediction decode step over B cached sequences.

    q: [B,g,H,D] codes of the g queries of one MTP step (positions n_b-g..n_b-1)
    q_scale: [B,g]; w: [B,g,H]; k: [B,Lmax,D] key cache codes; k_scale: [B,Lmax]
    cache_len: [B] int32 keys held per sequence, the g new keys included.
    """

    dtype: str
    B: int
    Lmax: int
    H: int
    D: int
    g: int
    q: np.ndarray
    q_scale: Optional[np.ndarray]
    w: np.ndarray
    k: np.ndarray
    k_scale: Optional[np.ndarray]
    cache_len: np.ndarray


# ----------------------------------------------------------------------------
# storage encoders (PyTorch CPU casts)
# ----------------------------------------------------------------------------

def encode_bf16(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _encode_fp8(x: np.ndarray) -> np.ndarray:
    x = np.clip(np.ascontiguousarray(x, dtype=np.float32), -448.0, 448.0)
    return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def encode_fp8_per_row(x: np.ndarray, row_axes: int):
    """Quantise with one float32 scale per leading index (the first `row_axes`
    axes); scale = amax/448 (1 for an all-zero row)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    lead = x.shape[:row_axes]
    flat = x.reshape(int(np.prod(lead)), -1)
    amax = np.abs(flat).max(axis=1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    codes = np.empty(flat.shape, np.uint8)
    step = max(1, (1 << 24) // max(1, flat.shape[1]))
    for i in range(0, flat.shape[0], step):
        codes[i:i + step] = _encode_fp8(flat[i:i + step] / scale[i:i + step, None])
    return codes.reshape(x.shape), scale.reshape(lead)


# ----------------------------------------------------------------------------
# generators
# ----------------------------------------------------------------------------

def _streams(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def tiny_integer(L=2048, H=4, D=32, seed=1001) -> PrefillInputs:
    """Small-integer bf16 inputs: q, k in {-4..4}/8, w in {1..4}/8.  Queries
    drift as a clipped random walk q_t = clip(q_{t-1} + {-1,0,1}/8, +-4/8) per
    element.  Every binary32 sum over these values is exact."""
    rq, rk, rw = _streams(seed, 3)
    steps = rq.integers(-1, 2, size=(L, H, D), dtype=np.int8)
    qi = np.empty((L, H, D), np.int8)
    cur = rq.integers(-4, 5, size=(H, D)).astype(np.int8)
    qi[0] = cur
    for t in range(1, L):
        cur = np.clip(cur + steps[t], -4, 4).astype(np.int8)
        qi[t] = cur
    ki = rk.integers(-4, 5, size=(L, D))
    wi = rw.integers(1, 5, size=(L, H))
    return PrefillInputs(
        dtype="bf16", L=L, H=H, D=D,
        q=encode_bf16(qi.astype(np.float32) / 8), q_scale=None,
        w=(wi.astype(np.float32) / 8),
        k=encode_bf16(ki.astype(np.float32) / 8), k_scale=None,
    )


def small_integer(L, H, D, seed, qmax=3, kmax=3, wmax=3, dtype="bf16") -> PrefillInputs:
    """Independent small integers (q, k in {-qmax..qmax}, w in {1..wmax}), for
    brute-force and invariant checks on tiny shapes.  For dtype="fp8" the
    integers are stored as E4M3FN codes with scale 1 (exact for |x| <= 16)."""
    rq, rk, rw = _streams(seed, 3)
    q = rq.integers(-qmax, qmax + 1, size=(L, H, D)).astype(np.float32)
    k = rk.integers(-kmax, kmax + 1, size=(L, D)).astype(np.float32)
    w = rw.integers(1, wmax + 1, size=(L, H)).astype(np.float32)
    if dtype == "bf16":
        return PrefillInputs("bf16", L, H, D, encode_bf16(q), None, w, encode_bf16(k), None)
    return PrefillInputs("fp8", L, H, D, _encode_fp8(q), np.ones(L, np.float32), w,
                         _encode_fp8(k), np.ones(L, np.float32))


def _random_walk_queries(rng, L, H, D, rho=0.95, sigma=0.05, chunk=4096):
    """Per head: q_0 = normalize(N(0,I)), q_t = normalize(rho*q_{t-1} + sigma*N(0,I))."""
    out = np.empty((L, H, D), np.float32)
    cur = rng.standard_normal((H, D), dtype=np.float32)
    cur /= np.linalg.norm(cur, axis=-1, keepdims=True)
    out[0] = cur
    rho = np.float32(rho)
    sigma = np.float32(sigma)
    for c0 in range(1, L, chunk):
        c1 = min(L, c0 + chunk)
        noise = rng.standard_normal((c1 - c0, H, D), dtype=np.float32)
        noise *= sigma
        for i in range(c1 - c0):
            cur = rho * cur + noise[i]
            cur /= np.sqrt(np.einsum("hd,hd->h", cur, cur))[:, None]
            out[c0 + i] = cur
    return out


def _lognormal_keys(rng, n, D, sigma=0.5):
    """k_s = s_s * N(0, I) with s_s ~ LogNormal(0, sigma): long-tailed key norms."""
    k = rng.standard_normal((n, D), dtype=np.float32)
    s = np.exp(np.float32(sigma) * rng.standard_normal(n, dtype=np.float32)).astype(np.float32)
    k *= s[:, None]
    return k


def dsa_prefill(L, H=64, D=128, dtype="bf16", seed=1002) -> PrefillInputs:
    """DSA-shaped prefill: random-walk queries (adjacent cosine about 0.86),
    log-normal key norms, w_h ~ U(0,1)/sqrt(H)."""
    rq, rk, rw = _streams(seed, 3)
    qf = _random_walk_queries(rq, L, H, D)
    kf = _lognormal_keys(rk, L, D)
    w = (rw.random((L, H), dtype=np.float32) / np.float32(np.sqrt(H))).astype(np.float32)
    if dtype == "bf16":
        return PrefillInputs("bf16", L, H, D, encode_bf16(qf), None, w, encode_bf16(kf), None)
    qc, qs = encode_fp8_per_row(qf, 1)
    kc, ks = encode_fp8_per_row(kf, 1)
    return PrefillInputs("fp8", L, H, D, qc, qs, w, kc, ks)


def decode_mtp(B=32, Lmin=32768, Lmax=131072, H=64, D=128, g=2, seed=1005,
               dtype="fp8") -> DecodeInputs:
    """MTP decode step: B sequences with cached-key lengths uniform in
    [Lmin, Lmax]; g queries per sequence (one token plus g-1 MTP tokens) drawn
    as g random-walk steps; keys as in dsa_prefill; w ~ U(0,1)/sqrt(H)."""
    rq, rk, rw, rl = _streams(seed, 4)
    cache_len = rl.integers(Lmin, Lmax + 1, size=B).astype(np.int32)
    cache_len = np.maximum(cache_len, g).astype(np.int32)
    qf = np.stack([_random_walk_queries(rq, g, H, D) for _ in range(B)])  # [B,g,H,D]
    w = (rw.random((B, g, H), dtype=np.float32) / np.float32(np.sqrt(H))).astype(np.float32)
    esz = np.uint16 if dtype == "bf16" else np.uint8
    k = np.zeros((B, Lmax, D), esz)
    k_scale = np.ones((B, Lmax), np.float32) if dtype == "fp8" else None
    for b in range(B):
        n = int(cache_len[b])
        kf = _lognormal_keys(rk, n, D)
        if dtype == "bf16":
            k[b, :n] = encode_bf16(kf)
        else:
            kc, ks = encode_fp8_per_row(kf, 1)
            k[b, :n] = kc
            k_scale[b, :n] = ks
    if dtype == "bf16":
        return DecodeInputs("bf16", B, Lmax, H, D, g, encode_bf16(qf), None, w, k, None, cache_len)
    qc, qs = encode_fp8_per_row(qf, 2)
    return DecodeInputs("fp8", B, Lmax, H, D, g, qc, qs, w, k, k_scale, cache_len)


@dataclass
class PagedCache:
    """A decode step's key cache laid out in pages of a shared pool.

    k_pages: [num_pages, page_size, D] codes; k_scale_pages: [num_pages,
    page_size] (fp8 only); block_table: [B, max_pages] int32, row b listing the
    pages that hold positions 0.., page_size at a time (-1 past them)."""

    page_size: int
    k_pages: np.ndarray
    k_scale_pages: Optional[np.ndarray]
    block_table: np.ndarray


def paged_cache(dec: DecodeInputs, page_size: int, seed: int = 2001,
                spare_pages: int = 3) -> PagedCache:
    """Scatter dec's key cache into pages of a pool in a random order, as a
    server's allocator leaves it.  Every byte that is not a cached key (the
    spare pages, the tail of each sequence's last page) holds random codes and
    random scales, so that a wrong page or a read past a sequence's end shows."""
    rng = np.random.Generator(np.random.PCG64(seed))
    npg = [(int(n) + page_size - 1) // page_size for n in dec.cache_len]
    max_pages = (dec.Lmax + page_size - 1) // page_size
    num_pages = sum(npg) + spare_pages
    perm = rng.permutation(num_pages).astype(np.int32)
    esz = dec.k.dtype
    kp = rng.integers(0, np.iinfo(esz).max, size=(num_pages, page_size, dec.D), dtype=esz,
                      endpoint=True)
    if dec.dtype == "bf16":  # random finite bf16 codes of moderate size
        kp &= np.uint16(0x807F)
        kp |= np.uint16(0x3E00)
    else:  # random finite E4M3FN codes (0x7F / 0xFF are NaN)
        kp[(kp & 0x7F) == 0x7F] &= np.uint8(0xF0)
    ksp = None
    if dec.k_scale is not None:
        ksp = rng.uniform(0.5, 2.0, size=(num_pages, page_size)).astype(np.float32)
    bt = np.full((dec.B, max_pages), -1, np.int32)
    used = 0
    for b in range(dec.B):
        n = int(dec.cache_len[b])
        for i in range(npg[b]):
            pg = int(perm[used])
            used += 1
            bt[b, i] = pg
            lo, hi = i * page_size, min(n, (i + 1) * page_size)
            kp[pg, : hi - lo] = dec.k[b, lo:hi]
            if ksp is not None:
                ksp[pg, : hi - lo] = dec.k_scale[b, lo:hi]
    return PagedCache(page_size, kp, ksp, bt)


# The five workloads: name -> (kind, parameters).
CONFIGS = {
    "tiny_prefill_2k": dict(kind="prefill", L=2048, H=4, D=32, g=4, topk=64, C=256,
                            dtype="bf16", gen="tiny_integer", seed=1001),
    "dsa_prefill_16k": dict(kind="prefill", L=16384, H=64, D=128, g=8, topk=2048, C=4096,
                            dtype="bf16", gen="dsa_prefill", seed=1002),
    "long_prefill_fp8_64k": dict(kind="prefill", L=65536, H=64, D=128, g=8, topk=2048,
                                 C=4096, dtype="fp8", gen="dsa_prefill", seed=1003),
    "prefill_128k": dict(kind="prefill", L=131072, H=64, D=128, g=8, topk=2048, C=4096,
                         dtype="bf16", gen="dsa_prefill", seed=1004, g_sweep=(4, 8, 16)),
    "decode_mtp_b32": dict(kind="decode", B=32, Lmin=32768, Lmax=131072, H=64, D=128, g=2,
                           topk=2048, C=4096, dtype="fp8", gen="decode_mtp", seed=1005),
}


def make(name: str, **override):
    """Build the inputs of a named workload (optionally overriding sizes)."""
    cfg = dict(CONFIGS[name])
    cfg.update(override)
    if cfg["gen"] == "tiny_integer":
        return tiny_integer(cfg["L"], cfg["H"], cfg["D"], cfg["seed"])
    if cfg["gen"] == "dsa_prefill":
        return dsa_prefill(cfg["L"], cfg["H"], cfg["D"], cfg["dtype"], cfg["seed"])
    return decode_mtp(cfg["B"], cfg["Lmin"], cfg["Lmax"], cfg["H"], cfg["D"], cfg["g"],
                      cfg["seed"], cfg["dtype"])
