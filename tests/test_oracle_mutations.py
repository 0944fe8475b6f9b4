"""Planted mistakes: each plausible error in the oracle fails at least one pin.

A mistake is planted by editing a copy of oracle/pivot_oracle.c (one textual
substitution), which is compiled with the oracle's own flags into a temporary
library.  The CPU pin suites then run against that library in a child process
(PIVOT_ORACLE_LIB names it) and must fail.  The unmodified copy must pass.
Nothing here touches the GPU or the HIP library.
"""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

import oracle
from conftest import ROOT

SRC = os.path.join(ROOT, "oracle", "pivot_oracle.c")
PIN_FILES = ["test_oracle_pins.py", "test_oracle_invariants.py", "test_oracle_attention.py",
             "test_oracle_paged.py", "test_oracle_proxy_division.py"]

# (name, text in pivot_oracle.c, replacement)
MUTATIONS = [
    ("scan only to the first member",
     "const int e = pos0 + n - 1 - excl;", "const int e = pos0 - excl;"),
    ("ReLU dropped",
     "double relu = dot > 0.0 ? dot : 0.0;", "double relu = dot;"),
    ("tie rule reversed",
     "return (a->pos > b->pos) - (a->pos < b->pos);", "return (a->pos < b->pos) - (a->pos > b->pos);"),
    ("Refine causal clip missing",
     "if (cand[j] >= 0 && cand[j] <= t) mpos[np++] = cand[j];", "if (cand[j] >= 0) mpos[np++] = cand[j];"),
    ("Reuse causal clip missing",
     "if (ptop[j] >= 0 && ptop[j] <= t) o[c++] = ptop[j];", "if (ptop[j] >= 0) o[c++] = ptop[j];"),
    ("proxy used to re-score in Refine",
     "score_keys(v, qc, row_scale(v, row0 + i), v->w + (long)(row0 + i) * H, mpos, np, msc);",
     "score_keys(v, pq, ps, pw, mpos, np, msc);"),
    ("mean divided by one member too many",
     "mean[e] = sum / (float)n;", "mean[e] = sum / (float)(n + 1);"),
    ("mean as a product with the reciprocal",
     "mean[e] = sum / (float)n;", "mean[e] = sum * (1.0f / (float)n);"),
    ("weights summed, not averaged",
     "w_out[h] = sum / (float)n;", "w_out[h] = sum;"),
    ("weight mean as a product with the reciprocal",
     "w_out[h] = sum / (float)n;", "w_out[h] = sum * (1.0f / (float)n);"),
    ("fp8 key scale dropped",
     "total = total * (double)qs * (double)v->k_scale[s];", "total = total * (double)qs;"),
    ("fp8 key scale of the previous key",
     "total = total * (double)qs * (double)v->k_scale[s];",
     "total = total * (double)qs * (double)v->k_scale[s > 0 ? s - 1 : s];"),
    ("fp8 proxy scale divisor",
     "float sp = amax > 0.0f ? amax / 448.0f : 1.0f;", "float sp = amax > 0.0f ? amax / 240.0f : 1.0f;"),
    ("one-member group re-quantised",
     "if (n == 1) {\n    size_t esz", "if (0) {\n    size_t esz"),
    ("dense row excludes itself",
     "int n = t + 1 > 0 ? t + 1 : 0;\n    double* sc", "int n = t > 0 ? t : 0;\n    double* sc"),
    ("head weight of the next head",
     "total += (double)w[h] * relu;", "total += (double)w[(h + 1) % H] * relu;"),
    ("key index shifted",
     "decode_codes(v->dtype, v->k, (long)s * v->D, v->D, kd);",
     "decode_codes(v->dtype, v->k, (long)(s > 0 ? s - 1 : s) * v->D, v->D, kd);"),
    ("e4m3 ties rounded up",
     "pick = (lo & 1) ? hi : lo;", "pick = hi;"),
    ("bf16 ties rounded up",
     "return (lo & 1u) ? hi : lo;", "return hi;"),
    ("window union without de-duplication",
     "if (c == 0 || all[i] != out[c - 1]) out[c++] = all[i];", "out[c++] = all[i];"),
    ("window starting one position late",
     "for (int s = t - W + 1; s <= t; ++s)", "for (int s = t - W + 2; s <= t; ++s)"),
    ("excluded window offset by one",
     "int t = rows[i] - excl;", "int t = rows[i] - excl + 1;"),
    ("attention denominator",
     "for (int c = 0; c < dv; ++c) o[c] /= den;", "for (int c = 0; c < dv; ++c) o[c] /= (den + 1.0);"),
]


def _build_variant(tmp, name, text):
    os.makedirs(tmp, exist_ok=True)
    src = os.path.join(tmp, "pivot_oracle.c")
    with open(src, "w") as f:
        f.write(text)
    hdr = os.path.join(ROOT, "oracle", "pivot_oracle.h")
    with open(hdr) as f, open(os.path.join(tmp, "pivot_oracle.h"), "w") as g:
        g.write(f.read())
    lib = os.path.join(tmp, "liboracle.so")
    subprocess.run(["gcc", *oracle.CFLAGS, "-o", lib, src, "-lm"], check=True,
                   capture_output=True)
    return lib


def _run_pins(lib):
    env = dict(os.environ, PIVOT_ORACLE_LIB=lib)
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
           *[os.path.join(ROOT, "tests", f) for f in PIN_FILES]]
    r = subprocess.run(cmd, env=env, capture_output=True, text=True, cwd=ROOT, timeout=600)
    return r.returncode, r.stdout[-2000:]


def test_every_planted_mistake_fails_a_pin():
    text = open(SRC).read()
    for name, old, new in MUTATIONS:
        assert text.count(old) == 1, f"{name}: the planted text must occur exactly once"
    with tempfile.TemporaryDirectory() as tmp:
        jobs = [("unmodified", text)] + [(name, text.replace(old, new)) for name, old, new in MUTATIONS]
        libs = [_build_variant(os.path.join(tmp, str(i)), n, t) for i, (n, t) in enumerate(jobs)]
        with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            results = list(ex.map(_run_pins, libs))
    rc0, out0 = results[0]
    assert rc0 == 0, f"the unmodified oracle must pass its pins:\n{out0}"
    survivors = [jobs[i][0] for i in range(1, len(jobs)) if results[i][0] == 0]
    assert not survivors, f"planted mistakes that no pin catches: {survivors}"
