"""The C ABI from plain C: tests/c/abi_host.c, compiled as C99 with gcc
against include/ffd.h and linked with the in-tree libffd.so, exercises the host
queries and the argument checks that precede any HIP call (no GPU needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_long_context_ffd_amd")


def test_c_program_uses_the_abi(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    if not os.path.exists(os.path.join(PKG, "libffd.so")):
        pytest.skip("libffd.so not built")
    exe = str(tmp_path / "abi_host")
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_host.c"), "-L", PKG, "-l:libffd.so", f"-Wl,-rpath,{PKG}", "-lm",
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
