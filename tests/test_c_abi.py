"""The C ABI from plain C (no GPU): tests/c_abi_check.c is compiled with the
host C compiler against include/dsa.h only, linked to the built libdsa.so and
run; it makes only calls that return before any device work."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "dynamic_sparse_attention_slash_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_header_and_library_from_c(tmp_path):
    if not os.path.exists(os.path.join(LIB_DIR, "libdsa.so")):
        pytest.fail("libdsa.so is not built (run __graft_entry__.build())")
    exe = str(tmp_path / "c_abi_check")
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi_check.c"), "-L", LIB_DIR, "-ldsa",
           "-Wl,-rpath," + LIB_DIR, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c abi: ok" in r.stdout
