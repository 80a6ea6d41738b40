"""The host allocator and planner under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only): a C++ stress driver through the C ABI."""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

from conftest import REPO

CSRC = os.path.join(REPO, "paged_kv_cache_123_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_pool_and_plan_under_asan_ubsan(tmp_path):
    exe = tmp_path / "pool_stress"
    srcs = [os.path.join(REPO, "tests", "cpp", "pool_stress.cpp")] + [
        os.path.join(CSRC, f) for f in ("block_pool.cpp", "sha256.cpp", "plan.cpp",
                                        "context_parallel.cpp", "status.cpp")]
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           f"-I{os.path.join(REPO, 'include')}", f"-I{CSRC}", *srcs, "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    # verify_asan_link_order=0: the environment may preload other libraries
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "pool_stress ok" in run.stdout
