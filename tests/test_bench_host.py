"""Host-side parts of bench.py (CPU only): the one-GPU contract and the
algorithmic work counts behind its roofline figures."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_proxy_scan_pairs_closed_form():
    # groups of g aligned at 0, group j scans keys 0..e_j with e_j = min(jg+g, L) - 1
    for L, g in ((131072, 8), (131072, 4), (131072, 16), (65536, 8), (16384, 8)):
        G = L // g
        assert bench.proxy_scan_pairs(L, g) == L * (G + 1) // 2
    # a partial last group and g = 1 (the dense scan: L(L+1)/2 pairs)
    assert bench.proxy_scan_pairs(10, 4) == 4 + 8 + 10
    assert bench.proxy_scan_pairs(2048, 1) == 2048 * 2049 // 2


def test_refine_pairs_small_cases():
    # every member of group j scores min(C, e_j + 1) candidates
    L, g, C = 10, 4, 5
    want = 4 * min(C, 4) + 4 * min(C, 8) + 2 * min(C, 10)
    assert bench.refine_pairs(L, g, C) == want
    # C covering every prefix: sum over members of their group's prefix length
    e = np.minimum((np.arange(3) + 1) * 4, L)
    n = np.array([4, 4, 2])
    assert bench.refine_pairs(L, g, 10 ** 6) == int((e * n).sum())


def test_work_counts_of_the_workloads():
    # the pair counts of the workloads' scope table (derived by counting)
    assert bench.proxy_scan_pairs(131072, 8) == 1_073_807_360
    assert bench.proxy_scan_pairs(131072, 4) == 2_147_549_184
    assert bench.proxy_scan_pairs(131072, 16) == 536_936_448
    assert bench.refine_pairs(131072, 8, 4096) == 528_498_688
    assert bench.proxy_scan_pairs(65536, 8) == 268_468_224
    assert bench.refine_pairs(65536, 8, 4096) == 260_063_232
    assert bench.proxy_scan_pairs(16384, 8) == 16_785_408
    assert bench.refine_pairs(16384, 8, 4096) == 58_736_640
