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


CLANG = "/opt/rocm/llvm/bin/clang"


@pytest.mark.skipif(not os.path.exists(CLANG), reason="no ROCm clang")
def test_host_code_under_address_and_ub_sanitizers(tmp_path):
    """The same C checks against a copy of the library whose host code is built
    with AddressSanitizer and UndefinedBehaviorSanitizer (device code as
    usual; any report aborts the run): the argument checks, workspace
    arithmetic and head-list handling touch no memory they do not own and do
    no undefined arithmetic, at the largest shapes the checks accept too."""
    from dynamic_sparse_attention_slash_amd import build as B
    lib = str(tmp_path / "libdsa.so")
    B.build(verbose=False, out=lib, sanitize=True)
    rt = os.path.dirname(subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                                        capture_output=True, text=True).stdout.strip())
    exe = str(tmp_path / "c_abi_check_san")
    cmd = [CLANG, "-std=c99", "-Wall", "-Werror", "-fsanitize=address,undefined", "-shared-libsan",
           "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi_check.c"), "-L", str(tmp_path), "-ldsa",
           "-Wl,-rpath," + str(tmp_path), "-Wl,-rpath," + rt, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c abi: ok" in r.stdout
