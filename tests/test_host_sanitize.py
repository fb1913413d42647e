"""The host-side validation layer (block geometry, keep rate, selection
and mixed-plan sizing, workspace layout) compiled by g++ with
AddressSanitizer and UndefinedBehaviorSanitizer and driven through every
error path by tests/host_check.cpp; no HIP and no GPU involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_validation_under_asan_ubsan(tmp_path):
    exe = tmp_path / "host_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "block_sparse_attention_centroids_amd", "csrc"),
           os.path.join(ROOT, "tests", "host_check.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "host checks ok" in r.stdout
