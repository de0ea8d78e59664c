"""The boundary is a plain C ABI: a C11 program that includes only
include/cpthd.h (compiled with gcc -std=c11 -pedantic -Werror, no HIP header)
links libcpthd.so and runs the calls that need no GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "thd_token_layout_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_program_links_and_runs(tmp_path):
    assert os.path.exists(os.path.join(PKG, "libcpthd.so")), "build the library first"
    exe = str(tmp_path / "c_consumer")
    rocm_lib = "/opt/rocm/lib"
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-pedantic", "-Werror",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_consumer.c"),
           "-L", PKG, "-lcpthd", f"-Wl,-rpath,{PKG}", f"-L{rocm_lib}", f"-Wl,-rpath-link,{rocm_lib}",
           f"-Wl,-rpath,{rocm_lib}", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "c consumer ok" in res.stdout
