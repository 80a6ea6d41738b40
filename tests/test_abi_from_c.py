"""The header is plain C and the library is usable from a C program (CPU only)."""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

from conftest import REPO

LIB_DIR = os.path.join(REPO, "paged_kv_cache_123_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_header_compiles_as_c99_and_c_program_runs(tmp_path):
    if not os.path.exists(os.path.join(LIB_DIR, "libpagedkv.so")):
        pytest.skip("library not built")
    exe = tmp_path / "abi_from_c"
    src = os.path.join(REPO, "tests", "c", "abi_from_c.c")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           f"-I{os.path.join(REPO, 'include')}", src, f"-L{LIB_DIR}", "-lpagedkv",
           f"-Wl,-rpath,{LIB_DIR}", "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "abi_from_c ok" in run.stdout
