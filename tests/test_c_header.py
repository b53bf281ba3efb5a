"""include/sfi.h is a C header: a C99 program compiles against it with gcc (warnings as
errors) and links libsfi.so; its validation-only calls run without a GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_kv_attention_dense_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_header_compiles_as_c_and_links(tmp_path):
    if not os.path.exists(os.path.join(PKG, "libsfi.so")):
        from sparse_kv_attention_dense_amd import build
        build.build()
    exe = str(tmp_path / "abi_from_c")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-isystem", "/opt/rocm/include",
           os.path.join(ROOT, "tests", "c", "abi_from_c.c"), "-L", PKG, "-lsfi",
           f"-Wl,-rpath,{PKG}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count(" ok") == 7, r.stdout
