"""The HIP-free host sources (LRU planner, q*, descriptor checks and layout,
host expert kernel) built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer and driven through their C ABI by
host_sanitize_main.cpp; any report fails the test (CPU only)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_expert_execution_amd", "csrc")
SOURCES = [os.path.join(CSRC, f) for f in ("host.cpp", "planner.cpp", "host_expert.cpp")]


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_sources_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_sanitize")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "host_sanitize_main.cpp")] + SOURCES + [
           "-lpthread", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-6000:]
    assert "host sanitize driver: ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
