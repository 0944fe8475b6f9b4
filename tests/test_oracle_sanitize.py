"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(host code only, gcc) and driven over many tiny shapes by
tests/oracle_sanitize_driver.c: any out-of-bounds access, use of freed memory,
leak, signed overflow or invalid shift in the oracle fails this test."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "oracle"),
           os.path.join(ROOT, "oracle", "pivot_oracle.c"),
           os.path.join(HERE, "oracle_sanitize_driver.c"), "-lm", "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr
    assert "oracle sanitizer driver: ok" in r.stdout
