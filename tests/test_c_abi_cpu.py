"""The C ABI from C: include/pagedkv.h compiles as strict C99, and a C program
linked against the built library drives the host entry points (allocator
walk-through of the pages, copy-on-write, precondition checks, argument
errors of device calls). No GPU is used."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "paged_kv_cache_316_amd")
LIB = os.path.join(PKG, "libpagedkv.so")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_host_entry_points_from_c(tmp_path):
    exe = tmp_path / "host_abi"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "host_abi.c"),
           "-L", PKG, "-l:libpagedkv.so", f"-Wl,-rpath,{PKG}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("0 failures")
    assert "FAIL" not in r.stdout
