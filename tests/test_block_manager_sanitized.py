"""The host block manager (csrc/pa_blocks.cpp) under AddressSanitizer and
UndefinedBehaviorSanitizer: a random-operation driver (tests/bm_random_ops.cpp)
checks its invariants after every step.  Host code only; no GPU involved."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_block_manager_random_ops_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = tmp_path / "bm_random_ops"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", f"-I{ROOT}/include", "-o", str(exe),
           os.path.join(ROOT, "tests", "bm_random_ops.cpp"),
           os.path.join(ROOT, "paged_kv_cache_275_amd", "csrc", "pa_blocks.cpp")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr or "").lower():
        pytest.skip("sanitizer runtime not available: " + r.stderr[-200:])
    assert r.returncode == 0, r.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, f"exit {run.returncode}\n{run.stdout}\n{run.stderr[-2000:]}"
    assert run.stdout.strip() == "ok"
