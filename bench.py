"""Benchmark of the PIVOT indexer on one MI355X.

One step = one call of the whole indexer hot path (proxy mean, full-prefix
proxy scan, proxy top-C, Refine gather-score, member top-k) on the 128K prefill
workload: L=131072, H=64, D=128, bf16, g=8, topk=2048, C=4096, inputs resident
in HBM.  Prints one JSON line:

  value      indexed queries/s = L / seconds per step
  roofline   the proxy scan kernel (the dominant kernel) against the bf16
             matrix-core peak, from HIP events on its launch stream
  cpu_baseline  the CPU oracle on a bounded sample of the same workload

plus context measured in the same run: speedup over the dense indexer (g=1)
on the same GPU, Refine/dense top-k overlap, the g sweep, PIVOT-Reuse, the
sliding window, several sequences in one call, the 16K bf16 and 64K fp8 prefill
workloads (with their scan's rate against the bf16 or fp8 matrix peak), the
MTP decode step (B=32, fp8, µs per step) and sparse main attention.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3]
    python bench.py --decode-only | --fp8-only | --attention-only   (one part alone)
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
FP8_PEAK_TFLOPS = 5000.0    # MI355X dense fp8 matrix peak
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E peak


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--g", type=int, default=8)
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the headline step (used under a profiler)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of the CPU-oracle baseline sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run 3 plain 1 GiB device copies (counter calibration)")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the MTP decode step (used under a profiler)")
    ap.add_argument("--fp8-only", action="store_true",
                    help="time only the 64K fp8 prefill workload (Reuse, Refine)")
    ap.add_argument("--attention-only", action="store_true",
                    help="time only the sparse main attention after the indexer")
    return ap.parse_args()


def upload(inp, torch):
    def codes(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).view(torch.float8_e4m3fn).cuda()

    def f32(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()

    d = dict(q=codes(inp.q), w=f32(inp.w), k=codes(inp.k), q_scale=f32(inp.q_scale),
             k_scale=f32(inp.k_scale))
    if hasattr(inp, "cache_len"):
        d["cache_len"] = torch.from_numpy(inp.cache_len.astype(np.int32)).cuda()
    return d


def time_steps(fn, steps, warmup, torch):
    """Median seconds per call over `steps` calls (after `warmup`), each call
    bracketed by two events on the current stream, the one the library
    launches on."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev])) / 1e3


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def measure_decode(torch, pv, synth, nd_steps, nd_prof):
    """The MTP decode step (B=32, g=2, fp8 cache of 32K-128K keys, Refine):
    microseconds per step without per-kernel events, then a profiled pass for
    the per-kernel times and the decode scan's HBM rate."""
    topk, C, H, D = 2048, 4096, 64, 128
    log("generating the decode inputs")
    dec = synth.make("decode_mtp_b32")
    dd = upload(dec, torch)
    B, Lmax = dec.B, dec.Lmax
    dws = torch.empty(max(pv.decode_workspace_size(B, Lmax, H, D, 2, topk, C, m, 1)
                          for m in ("refine", "dense")), dtype=torch.uint8, device="cuda")
    dout = torch.empty((B, 2, topk), dtype=torch.int32, device="cuda")

    def dstep(mode="refine"):
        pv.indexer_decode(dd["q"], dd["w"], dd["k"], dd["cache_len"], topk=topk, C=C,
                          mode=mode, q_scale=dd["q_scale"], k_scale=dd["k_scale"], out=dout,
                          workspace=dws)

    dsec = time_steps(dstep, nd_steps, 10, torch)
    # a plain device copy of the whole key-cache buffer (bytes read + bytes
    # written per second), as a measured stream rate beside the 8 TB/s
    # datasheet peak
    kview = dd["k"].view(torch.uint8)
    kcopy = torch.empty_like(kview)
    stream_sec = time_steps(lambda: kcopy.copy_(kview), 20, 3, torch)
    stream_gbs = 2 * kview.numel() / stream_sec / 1e9
    del kcopy
    pv.profile_enable(True)
    pv.profile_read()
    for _ in range(nd_prof):
        dstep()
    torch.cuda.synchronize()
    dprof = pv.profile_read()
    pv.profile_enable(False)
    key_bytes = float(dec.cache_len.astype(np.int64).sum()) * (D + 4)
    scan_ms_d = dprof["decode_scan"][0] / nd_prof
    dense_dsec = time_steps(lambda: dstep("dense"), nd_steps, 5, torch)
    # the same step over a paged cache: 64-key pages of a shuffled pool
    log("laying the decode cache out in 64-key pages")
    pc = synth.paged_cache(dec, 64)
    kp = torch.from_numpy(pc.k_pages).view(torch.float8_e4m3fn).cuda()
    ksp = torch.from_numpy(pc.k_scale_pages).cuda()
    btd = torch.from_numpy(pc.block_table).cuda()

    def pstep():
        pv.indexer_decode_paged(dd["q"], dd["w"], kp, btd, dd["cache_len"], topk=topk, C=C,
                                mode="refine", q_scale=dd["q_scale"], k_scale=ksp, out=dout,
                                workspace=dws)

    paged_sec = time_steps(pstep, nd_steps, 10, torch)
    pv.profile_enable(True)
    pv.profile_read()
    for _ in range(nd_prof):
        pstep()
    torch.cuda.synchronize()
    pprof = pv.profile_read()
    pv.profile_enable(False)
    pscan_ms = pprof["decode_scan"][0] / nd_prof
    del kp, ksp, btd, pc
    # a deeper multi-token-prediction group: four queries per sequence, same
    # cache lengths and distributions
    del dd, dws, dout
    torch.cuda.empty_cache()
    dec4 = synth.make("decode_mtp_b32", g=4)
    dd4 = upload(dec4, torch)
    ws4 = torch.empty(pv.decode_workspace_size(B, Lmax, H, D, 4, topk, C, "refine", 1),
                      dtype=torch.uint8, device="cuda")
    out4 = torch.empty((B, 4, topk), dtype=torch.int32, device="cuda")
    g4_sec = time_steps(lambda: pv.indexer_decode(dd4["q"], dd4["w"], dd4["k"], dd4["cache_len"],
                                                  topk=topk, C=C, mode="refine",
                                                  q_scale=dd4["q_scale"], k_scale=dd4["k_scale"],
                                                  out=out4, workspace=ws4),
                        nd_steps, 5, torch)
    del dd4, ws4, out4
    res = {
        "workload": "decode_mtp_b32 (B=32, g=2, fp8, cache 32K-128K)",
        "us_per_step": dsec * 1e6,
        "dense_us_per_step": dense_dsec * 1e6,
        "refine_g4_us_per_step": g4_sec * 1e6,
        "paged64_us_per_step": paged_sec * 1e6,
        "paged64_decode_scan_us": pscan_ms * 1e3,
        "paged64_decode_scan_hbm_GBs": key_bytes / (pscan_ms / 1e3) / 1e9,
        "paged64_refine_us": pprof["refine_score"][0] / nd_prof * 1e3,
        "key_stream_bytes": key_bytes,
        "decode_scan_us": scan_ms_d * 1e3,
        "decode_scan_hbm_GBs": key_bytes / (scan_ms_d / 1e3) / 1e9,
        "decode_scan_hbm_frac": key_bytes / (scan_ms_d / 1e3) / 1e9 / HBM_PEAK_GBS,
        "stream_copy_GBs": stream_gbs,
        "stream_copy_source": f"device copy of the {kview.numel() / 2**20:.0f} MiB key-cache buffer, read + "
                              "written bytes per second (measured, not the datasheet peak)",
        "decode_scan_frac_of_stream_copy": key_bytes / (scan_ms_d / 1e3) / 1e9 / stream_gbs,
        "kernels_us": {k: v[0] / nd_prof * 1e3 for k, v in dprof.items() if v[1]},
    }
    log(f"decode {dsec*1e6:.1f} us/step; scan {key_bytes/(scan_ms_d/1e3)/1e9:.0f} GB/s; "
        f"g=4 {g4_sec*1e6:.1f} us/step; paged (64) {paged_sec*1e6:.1f} us/step, "
        f"scan {pscan_ms*1e3:.1f} us")
    torch.cuda.empty_cache()
    return res


def measure_prefill(torch, pv, d, L, modes, peak, g=8, topk=2048, C=4096, steps=10):
    """ms per call and queries/s of one prefill workload (g=8 groups; dense is
    g=1), and the full-prefix scan's matrix-core rate from the library's
    per-launch events against `peak` (the code type's dense peak)."""
    H, D = d["q"].shape[1], d["q"].shape[2]
    fp8 = d.get("q_scale") is not None
    res = {"L": L, "H": H, "D": D, "dtype": "fp8" if fp8 else "bf16", "g": g, "topk": topk, "C": C}
    out = torch.empty((L, topk), dtype=torch.int32, device="cuda")
    for mode in modes:
        gg, cc = (1, topk) if mode == "dense" else (g, C)
        ws = torch.empty(pv.workspace_size(L, H, D, gg, topk, cc, mode, 1 if fp8 else 0),
                         dtype=torch.uint8, device="cuda")
        f = lambda: pv.indexer(d["q"], d["w"], d["k"], g=gg, topk=topk, C=cc, mode=mode, out=out,
                               workspace=ws, q_scale=d.get("q_scale"), k_scale=d.get("k_scale"))
        s = time_steps(f, steps, 3, torch)
        pv.profile_enable(True)
        pv.profile_read()
        f()
        torch.cuda.synchronize()
        prof = pv.profile_read()
        pv.profile_enable(False)
        scan_tf = 2.0 * H * D * proxy_scan_pairs(L, gg) / (prof["scan"][0] / 1e3) / 1e12
        res[mode] = {"ms_per_call": s * 1e3, "queries_per_s": L / s, "scan_TFLOPs": scan_tf,
                     "scan_frac_of_peak": scan_tf / peak,
                     "kernels_ms": {k: v[0] for k, v in prof.items() if v[1]}}
        del ws
    if "dense" in res:
        for mode in modes:
            if mode != "dense":
                res[mode]["speedup_vs_dense"] = res["dense"]["ms_per_call"] / res[mode]["ms_per_call"]
    log(f"prefill L={L} {res['dtype']}: " + ", ".join(f"{m} {res[m]['ms_per_call']:.2f} ms" for m in modes))
    del out
    torch.cuda.empty_cache()
    return res


def measure_attention(torch, pv, synth):
    """Sparse main attention after the indexer (multi-query, 64 heads,
    d = dv = 128, bf16 keys and values): the B=32 decode step on the decode
    workload's Refine rows, and the 16K prefill on its Refine rows.  Reports
    time, the bytes of key and value rows the selected positions gather, and
    the matrix-core work 2 * Hq * (d + dv) per selected position."""
    Hq, d = 64, 128
    res = {}
    gen = torch.Generator(device="cuda").manual_seed(1234)
    # decode: Refine rows of the decode workload
    dec = synth.make("decode_mtp_b32")
    dd = upload(dec, torch)
    B, Lmax, g = dec.B, dec.Lmax, dec.g
    rows = pv.indexer_decode(dd["q"], dd["w"], dd["k"], dd["cache_len"], topk=2048, C=4096,
                             mode="refine", q_scale=dd["q_scale"], k_scale=dd["k_scale"])
    del dd
    idx = rows.reshape(B * g, 2048).contiguous()
    kc = torch.randn((B, Lmax, d), generator=gen, device="cuda").to(torch.bfloat16)
    vc = torch.randn((B, Lmax, d), generator=gen, device="cuda").to(torch.bfloat16)
    qa = torch.randn((B * g, Hq, d), generator=gen, device="cuda").to(torch.bfloat16)
    out = torch.empty((B * g, Hq, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(256, pv.load().pivot_sparse_attention_workspace_size(B * g, Hq, d, 2048)),
                     dtype=torch.uint8, device="cuda")
    f = lambda: pv.sparse_attention(qa, kc, vc, idx, rows_per_seq=g, out=out, workspace=ws)
    sec = time_steps(f, 200, 10, torch)
    nsel = float((idx >= 0).sum().item())
    gb = nsel * 2 * d * 2 + qa.numel() * 2 + out.numel() * 4
    res["decode_b32"] = {"us_per_step": sec * 1e6, "selected_positions": nsel,
                         "bytes": gb, "GBs": gb / sec / 1e9, "hbm_frac": gb / sec / 1e9 / HBM_PEAK_GBS}
    del kc, vc, qa, out, ws, idx, rows
    torch.cuda.empty_cache()
    # prefill: Refine rows of the 16K workload
    inp = synth.make("dsa_prefill_16k")
    dp = upload(inp, torch)
    L = inp.L
    rows = pv.indexer(dp["q"], dp["w"], dp["k"], g=8, topk=2048, C=4096, mode="refine")
    del dp
    kp = torch.randn((L, d), generator=gen, device="cuda").to(torch.bfloat16)
    vp = torch.randn((L, d), generator=gen, device="cuda").to(torch.bfloat16)
    qp = torch.randn((L, Hq, d), generator=gen, device="cuda").to(torch.bfloat16)
    out = torch.empty((L, Hq, d), dtype=torch.float32, device="cuda")
    f = lambda: pv.sparse_attention(qp, kp, vp, rows, out=out)
    sec = time_steps(f, 10, 3, torch)
    nsel = float((rows >= 0).sum().item())
    fl = 2.0 * Hq * 2 * d * nsel
    res["prefill_16k"] = {"ms_per_call": sec * 1e3, "selected_positions": nsel,
                          "TFLOPs": fl / sec / 1e12, "mfma_frac": fl / sec / 1e12 / BF16_PEAK_TFLOPS}
    log(f"sparse attention: decode {res['decode_b32']['us_per_step']:.1f} us "
        f"({res['decode_b32']['GBs']:.0f} GB/s), prefill 16K {sec*1e3:.2f} ms "
        f"({fl/sec/1e12:.0f} TFLOP/s)")
    del kp, vp, qp, out, rows
    torch.cuda.empty_cache()
    return res


# Sources of the full-prefix scan kernel: the HBM bytes measured with
# rocprofv3 counters (FETCH_SIZE, WRITE_SIZE, calibrated on a plain copy) are
# reported only while these files are unchanged since the measurement.
SCAN_SOURCES = ("pivot_device.h", "pivot_kernels.h", "pivot_score.h", "pivot_score_launch.h",
                "score_bf16.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_128k_refine_g8_hbm_counters.md")


def scan_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in SCAN_SOURCES:
        with open(os.path.join(ROOT, "top_token_selection_pivot_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic():
    """HBM bytes per scan launch from the committed counter summary, or None
    when it is missing or the scan's sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            for line in fh:
                if line.startswith("scan-traffic:"):
                    f = dict(kv.split("=") for kv in line.split(":", 1)[1].split())
                    if f.get("sources") == scan_source_hash():
                        return {"fetch_bytes": float(f["fetch"]), "write_bytes": float(f["write"]),
                                "bytes": float(f["fetch"]) + float(f["write"]),
                                "per": "launch", "source": os.path.basename(TRAFFIC_FILE)}
    except (OSError, ValueError, KeyError):
        pass
    return None


def proxy_scan_pairs(L, g):
    """sum over groups j of (e_j + 1): keys scanned by the proxies."""
    G = (L + g - 1) // g
    e = np.minimum((np.arange(G, dtype=np.int64) + 1) * g, L)
    return int(e.sum())


def refine_pairs(L, g, C):
    G = (L + g - 1) // g
    first = np.arange(G, dtype=np.int64) * g
    n = np.minimum(first + g, L) - first
    e = first + n
    return int((np.minimum(C, e) * n).sum())


def cpu_baseline(inp, g, topk, C, budget_s):
    """The oracle (single-threaded C) on whole Refine groups of the same
    workload until the time budget is spent; returns queries/s."""
    import oracle
    v = oracle.View.of(inp)
    G = (inp.L + g - 1) // g
    rng = np.random.default_rng(0)
    order = rng.permutation(G)
    done_q = 0
    groups = []
    t0 = time.perf_counter()
    for j in order:
        oracle.prefill_groups(v, inp.L, g, topk, C, "refine", [int(j)])
        done_q += min(g, inp.L - int(j) * g)
        groups.append(int(j))
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return done_q / dt, dt, groups


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: the indexer path here is built and measured "
              "on one MI355X (no multi-GPU path); use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    import top_token_selection_pivot_amd as pv

    pv.load()
    if args.calibrate_copy:
        # a plain copy of known size: 1 GiB read + 1 GiB written per dispatch
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
        torch.cuda.empty_cache()
    if args.decode_only:
        res = measure_decode(torch, pv, synth, args.steps, args.steps)
        print(json.dumps({"metric": "decode us/step (MTP, B=32, g=2, fp8, Refine)",
                          "value": res["us_per_step"], "unit": "us/step", "n_gpus": 1,
                          "steps": args.steps, "higher_is_better": False, "decode": res}),
              flush=True)
        return
    if args.fp8_only:
        log("generating the 64K fp8 prefill inputs")
        d8 = upload(synth.make("long_prefill_fp8_64k"), torch)
        res = measure_prefill(torch, pv, d8, 65536, ("reuse", "refine"), FP8_PEAK_TFLOPS,
                              steps=args.steps)
        print(json.dumps({"metric": "64K fp8 prefill ms/call (g=8)", "n_gpus": 1,
                          "long_prefill_fp8_64k": res}), flush=True)
        return
    if args.attention_only:
        res = measure_attention(torch, pv, synth)
        print(json.dumps({"metric": "sparse attention after the indexer", "n_gpus": 1,
                          "sparse_attention": res}), flush=True)
        return
    L, H, D, g, topk, C = 131072, 64, 128, args.g, 2048, 4096
    log("generating the 128K prefill inputs")
    inp = synth.make("prefill_128k")
    d = upload(inp, torch)
    ws = torch.empty(pv.workspace_size(L, H, D, g, topk, C, "refine", 0), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((L, topk), dtype=torch.int32, device="cuda")

    def step():
        pv.indexer(d["q"], d["w"], d["k"], g=g, topk=topk, C=C, mode="refine", out=out,
                   workspace=ws)

    log(f"timing PIVOT-Refine g={g}: {args.warmup} warmup + {args.steps} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    pv.profile_enable(True)
    pv.profile_read()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / args.steps
    prof = pv.profile_read()
    pv.profile_enable(False)
    ms_step = sec * 1e3
    qps = L / sec
    scan_ms, scan_n = prof["scan"]
    flops = 2.0 * H * D * proxy_scan_pairs(L, g) * args.steps
    achieved = flops / (scan_ms / 1e3) / 1e12
    kern = {k: {"ms_per_step": v[0] / args.steps, "launches_per_step": v[1] / args.steps}
            for k, v in prof.items() if v[1]}
    log(f"refine g={g}: {ms_step:.2f} ms/step, {qps:,.0f} queries/s; scan {achieved:.0f} TFLOP/s")

    result = {
        "metric": "indexed queries/s at L=128K prefill (PIVOT-Refine g=8)",
        "value": qps,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random-walk queries, log-normal keys)",
        "config": {"workload": "prefill_128k", "L": L, "H": H, "D": D, "g": g, "topk": topk,
                   "C": C, "mode": "refine"},
        "roofline": {
            "kernel": "scan (proxy full-prefix scan)",
            "bound": "mfma",
            "achieved": achieved,
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / BF16_PEAK_TFLOPS,
            "traffic": committed_traffic(),
            "launches_per_step": scan_n / args.steps,
            "avg_launch_ms": scan_ms / max(1, scan_n),
            "algorithmic_flops_per_step": 2.0 * H * D * proxy_scan_pairs(L, g),
        },
        "kernels": kern,
    }

    if not args.no_extras:
        extras = {}
        # dense indexer (g = 1) on the same inputs: our own baseline kernel
        ws_d = torch.empty(pv.workspace_size(L, H, D, 1, topk, topk, "dense", 0),
                           dtype=torch.uint8, device="cuda")
        out_d = torch.empty((L, topk), dtype=torch.int32, device="cuda")
        log("timing the dense indexer")
        sec_d = time_steps(lambda: pv.indexer(d["q"], d["w"], d["k"], g=1, topk=topk, C=topk,
                                              mode="dense", out=out_d, workspace=ws_d),
                           10, 2, torch)
        extras["dense_ms_per_step"] = sec_d * 1e3
        extras["dense_queries_per_s"] = L / sec_d
        extras["refine_speedup_vs_dense"] = sec_d / sec
        # per-query top-k overlap of Refine with dense (all rows, on device)
        step()
        torch.cuda.synchronize()
        dense_rows = out_d.to(torch.int64)
        ref_rows = out.to(torch.int64)
        big = torch.iinfo(torch.int64).max
        dsort = torch.where(dense_rows < 0, torch.full_like(dense_rows, big), dense_rows)
        idx = torch.searchsorted(dsort, ref_rows).clamp_(max=topk - 1)
        hit = (dsort.gather(1, idx) == ref_rows) & (ref_rows >= 0)
        nd = (dense_rows >= 0).sum(1).clamp_(min=1)
        ov = (hit.sum(1).double() / nd.double()).cpu().numpy()
        extras["refine_overlap_with_dense"] = {"mean": float(ov.mean()),
                                               "p5": float(np.percentile(ov, 5)),
                                               "min": float(ov.min())}
        adj = (dsort[1:].gather(1, torch.searchsorted(dsort[1:], dense_rows[:-1]).clamp_(max=topk - 1))
               == dense_rows[:-1]) & (dense_rows[:-1] >= 0)
        extras["dense_adjacent_query_overlap"] = float((adj.sum(1).double() / topk).mean())
        del dense_rows, ref_rows, dsort, idx, hit, adj
        del out_d, ws_d
        torch.cuda.empty_cache()
        # g sweep and Reuse
        sweep = {}
        for gg in (4, 8, 16):
            ws_g = torch.empty(pv.workspace_size(L, H, D, gg, topk, 2 * topk, "refine", 0),
                               dtype=torch.uint8, device="cuda")
            s = time_steps(lambda: pv.indexer(d["q"], d["w"], d["k"], g=gg, topk=topk,
                                              C=2 * topk, mode="refine", out=out, workspace=ws_g),
                           10, 3, torch)
            sweep[f"refine_g{gg}"] = {"ms_per_step": s * 1e3, "queries_per_s": L / s,
                                      "speedup_vs_dense": sec_d / s}
        s = time_steps(lambda: pv.indexer(d["q"], d["w"], d["k"], g=8, topk=topk, C=C,
                                          mode="reuse", out=out, workspace=ws), 10, 3, torch)
        sweep["reuse_g8"] = {"ms_per_step": s * 1e3, "queries_per_s": L / s,
                             "speedup_vs_dense": sec_d / s}
        extras["g_sweep"] = sweep
        # sliding window added to the selection (both designs), Refine g=8
        W = 128
        out_w = torch.empty((L, topk + W), dtype=torch.int32, device="cuda")
        win = {"window": W}
        for wm in ("shared", "excluded"):
            f = lambda: pv.indexer(d["q"], d["w"], d["k"], g=g, topk=topk, C=C, mode="refine",
                                   out=out_w, workspace=ws, window=W, window_mode=wm)
            s = time_steps(f, 10, 3, torch)
            pv.profile_enable(True)
            pv.profile_read()
            f()
            torch.cuda.synchronize()
            prof = pv.profile_read()
            pv.profile_enable(False)
            wms, wn = prof["window"]
            # the union reads each row's selection (topk entries) and writes
            # the rest of the row: (topk + topk + W) * 4 bytes per row at most
            ub = L * (2 * topk + W) * 4
            win[wm] = {"ms_per_step": s * 1e3, "queries_per_s": L / s,
                       "union_kernel_ms": wms / max(1, wn), "union_kernel_GBs": ub / (wms / max(1, wn)) / 1e6}
        extras["window_refine_g8"] = win
        del out_w
        log(f"dense {sec_d*1e3:.1f} ms; speedup {sec_d/sec:.2f}x; overlap {ov.mean():.4f}")
        del d, ws, out
        torch.cuda.empty_cache()

        # several sequences of different lengths in one call (Refine g=8): the
        # 16K workload's distributions, cut into sequences of 8K, 4K, 2K, 1K, 512, 256, 256
        inp_v = synth.make("dsa_prefill_16k")
        dv_ = upload(inp_v, torch)
        lens = [8192, 4096, 2048, 1024, 512, 256, 256]
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        out_v = torch.empty((16384, topk), dtype=torch.int32, device="cuda")
        s_v = time_steps(lambda: pv.indexer_varlen(dv_["q"], dv_["w"], dv_["k"], cu, g=8, topk=topk, C=C,
                                                   mode="refine", out=out_v), 10, 3, torch)
        extras["varlen_refine_g8"] = {"lengths": lens, "ms_per_call": s_v * 1e3,
                                      "queries_per_s": 16384 / s_v}
        del out_v
        # cross-layer index reuse stacked on the indexer: four layers of the
        # 16K workload's shape (each its own seeded inputs), every layer full
        # against every other layer reusing the one before it
        layer_in = [dv_] + [upload(synth.make("dsa_prefill_16k", seed=2101 + l), torch) for l in range(3)]
        louts = [torch.empty((16384, topk), dtype=torch.int32, device="cuda") for _ in range(4)]
        ws_l = torch.empty(pv.workspace_size(16384, H, D, 8, topk, C, "refine", 0), dtype=torch.uint8,
                           device="cuda")
        ic = {"layers": 4, "workload": "dsa_prefill_16k per layer, Refine g=8"}
        for name, full in (("all_full", [1, 1, 1, 1]), ("alternate", [1, 0, 1, 0])):
            f = lambda full=full: pv.indexer_layers([x["q"] for x in layer_in], [x["w"] for x in layer_in],
                                                    [x["k"] for x in layer_in], full=full, g=8, topk=topk, C=C,
                                                    mode="refine", outs=louts, workspace=ws_l)
            s = time_steps(f, 10, 3, torch)
            ic[name] = {"full": full, "ms_per_step": s * 1e3}
        pv.profile_enable(True)
        pv.profile_read()
        pv.indexer_layers([x["q"] for x in layer_in], [x["w"] for x in layer_in], [x["k"] for x in layer_in],
                          full=[1, 0, 1, 0], g=8, topk=topk, C=C, mode="refine", outs=louts, workspace=ws_l)
        torch.cuda.synchronize()
        lp = pv.profile_read()
        pv.profile_enable(False)
        cms, cn = lp["layer_copy"]
        ic["copy_kernel_us"] = cms / max(1, cn) * 1e3
        ic["copy_kernel_GBs"] = 2 * 16384 * topk * 4 / (cms / max(1, cn) / 1e3) / 1e9
        ic["speedup"] = ic["all_full"]["ms_per_step"] / ic["alternate"]["ms_per_step"]
        extras["index_cache_16k"] = ic
        log(f"index reuse, 4 layers of 16K: all full {ic['all_full']['ms_per_step']:.2f} ms, "
            f"alternate {ic['alternate']['ms_per_step']:.2f} ms; copy {ic['copy_kernel_GBs']:.0f} GB/s")
        del layer_in, louts, ws_l
        # the other prefill workloads, one sequence each: 16K bf16 (dense,
        # Reuse, Refine) and 64K fp8 (Reuse, Refine)
        other = {"dsa_prefill_16k": measure_prefill(torch, pv, dv_, 16384, ("dense", "reuse", "refine"),
                                                    BF16_PEAK_TFLOPS)}
        del dv_
        torch.cuda.empty_cache()
        log("generating the 64K fp8 prefill inputs")
        d8 = upload(synth.make("long_prefill_fp8_64k"), torch)
        other["long_prefill_fp8_64k"] = measure_prefill(torch, pv, d8, 65536, ("reuse", "refine"),
                                                        FP8_PEAK_TFLOPS)
        extras["other_prefill_workloads"] = other
        del d8
        torch.cuda.empty_cache()
        extras["decode"] = measure_decode(torch, pv, synth, 200, 100)
        extras["sparse_attention"] = measure_attention(torch, pv, synth)
        extras["pages_claims_context"] = ("up to 4x indexer speedup, about 3x for Refine, "
                                          "1.6x end-to-end on DeepSeek-V3.2/GLM-5.1; "
                                          "no hardware stated")
        result["extras"] = extras

        log(f"CPU oracle baseline (~{args.cpu_seconds:.0f} s)")
        cqps, cdt, groups = cpu_baseline(inp, g, topk, C, args.cpu_seconds)
        result["cpu_baseline"] = {
            "value": cqps, "unit": "queries/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(groups)} whole Refine groups (g={g}, {len(groups)*g} queries) of "
                      f"the 128K workload, seeded-random group order, {cdt:.1f} s single-threaded",
            "host": cpu_model(),
            "host_threads_available": os.cpu_count(),
            "extrapolated_full_call_s": inp.L / cqps,
            "extrapolation": "L / (sampled queries/s); the sampled groups lie in seeded-random "
                             "order over the whole sequence",
        }

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
