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


@pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None, reason="gcc/g++ not available")
def test_host_validation_under_sanitizers(tmp_path):
    """The host layer (abi.cpp, every argument check of every entry point) built
    with AddressSanitizer and UBSan, the launch functions replaced by stand-ins
    that report an error, and driven by tests/c_validation_fuzz.c: seeded random
    arguments (integer edge values, NULL and fake pointers) through every entry
    point; every call returns a known status, with no memory error, leak or
    undefined behaviour (an int32 overflow in the size helpers was found this way)."""
    rocm_inc, rocm_lib = "/opt/rocm/include", "/opt/rocm/lib"
    if not os.path.exists(os.path.join(rocm_lib, "libamdhip64.so")):
        pytest.skip("HIP runtime library not found")
    san = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"), "-I", rocm_inc,
           "-D__HIP_PLATFORM_AMD__"]
    objs = []
    for src in (os.path.join(PKG, "csrc", "abi.cpp"), os.path.join(ROOT, "tests", "abi_stubs.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-fPIC", "-Wall", *san, *inc, "-c", src, "-o", obj],
                       check=True, capture_output=True, text=True)
        objs.append(obj)
    lib = str(tmp_path / "libcpthd_san.so")
    subprocess.run(["g++", "-shared", "-fPIC", *san, *objs, f"-L{rocm_lib}", "-lamdhip64",
                    f"-Wl,-rpath,{rocm_lib}", "-o", lib], check=True, capture_output=True, text=True)
    exe = str(tmp_path / "fuzz")
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-Wall", "-Wextra", "-pedantic", "-Werror", *san,
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_validation_fuzz.c"),
                    f"-L{tmp_path}", "-lcpthd_san", f"-Wl,-rpath,{tmp_path}", f"-L{rocm_lib}",
                    f"-Wl,-rpath-link,{rocm_lib}", "-o", exe], check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    for seed in ("0", "1", "2"):
        res = subprocess.run([exe, seed, "20000"], capture_output=True, text=True, timeout=300, env=env)
        assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
        assert "fuzz ok" in res.stdout


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="hipcc not available")
@pytest.mark.parametrize("flags", [["-O0", "-fwrapv"], ["-O2"]], ids=["O0-wrapv", "O2"])
def test_find_doc_near_int32_max(tmp_path, flags):
    """The document search of the permutation and metadata kernels, built for the
    host, at document counts up to 2^31 - 1 (tables computed on the fly).  With
    wrapping int32 arithmetic the former midpoint (lo + hi + 1) / 2 overflowed and
    the search never ended; the timeout turns such a hang into a failure."""
    exe = str(tmp_path / "find_doc_host")
    subprocess.run(["/opt/rocm/bin/hipcc", "-x", "hip", "--cuda-host-only", "-std=c++17", *flags,
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
                    os.path.join(ROOT, "tests", "find_doc_host.hip"), "-o", exe],
                   check=True, capture_output=True, text=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0 and "find_doc ok" in res.stdout, res.stdout + res.stderr


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="hipcc not available")
def test_row_chunk_index_arithmetic(tmp_path):
    """The row-chunk kernel's index arithmetic (chunk_map.h), built for the host and run
    over whole grids: every workgroup's row and chunk, every row's rank, local row and
    global row against plain division and the ownership formula, all in range, each
    global row written once; the magic-number division at edge and random arguments."""
    exe = str(tmp_path / "chunk_map_host")
    subprocess.run(["/opt/rocm/bin/hipcc", "-x", "hip", "--cuda-host-only", "-std=c++17", "-O2",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
                    os.path.join(ROOT, "tests", "chunk_map_host.hip"), "-o", exe],
                   check=True, capture_output=True, text=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=240)
    assert res.returncode == 0 and "chunk_map ok" in res.stdout, res.stdout + res.stderr
