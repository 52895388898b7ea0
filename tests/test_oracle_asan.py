"""The C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (host code only, gcc)
and run over every flag combination, packed and batched sequences, empty segments, absent
h0/hT and the decode step (tests/asan_oracle_driver.c). Any out-of-bounds access, leak or
undefined behaviour fails the run."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_address_sanitizer(tmp_path):
    exe = str(tmp_path / "asan_oracle")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           os.path.join(ROOT, "oracle", "gdr_oracle.c"), os.path.join(ROOT, "tests", "asan_oracle_driver.c"),
           "-o", exe, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in r.stderr.lower() and "cannot find" in r.stderr.lower():
        pytest.skip("libasan is not installed: " + r.stderr.strip()[-200:])
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", OMP_NUM_THREADS="2")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0 and "asan driver ok" in run.stdout, run.stdout + run.stderr
