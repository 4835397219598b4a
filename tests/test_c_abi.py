"""The C ABI from a plain C99 program (CPU only): include/var_attn.h compiles
as C with warnings as errors, links against libvarattn.so, and the host-only
calls behave (extent, mask dimensions, split plan, status strings, argument
errors that return before any HIP call)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c99_client(tmp_path):
    from scale_wise_attention_amd import api
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path / "abi_check")
    libdir = os.path.dirname(api.LIB_PATH)
    cmd = [cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi", "abi_check.c"), "-o", exe, "-L", libdir, "-lvarattn",
           f"-Wl,-rpath,{libdir}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "c abi: ok" in r.stdout, r.stdout + r.stderr
