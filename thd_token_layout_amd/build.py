"""Build libcpthd.so (HIP kernels for gfx950 + the C-ABI layer) in-tree.

    python -m thd_token_layout_amd.build          # or: python thd_token_layout_amd/build.py

Compiles every time it is called.  Outputs: thd_token_layout_amd/libcpthd.so
(the library) and thd_token_layout_amd/libcpthd_roofline.so (plain streaming
kernels the benchmark measures the chip's ceiling with; not part of the
library).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libcpthd.so")
ROOFLINE_LIB = os.path.join(PKG, "libcpthd_roofline.so")
ROOFLINE_SOURCE = "roofline.hip"

ARCH = "gfx950"
HIP_SOURCES = ["meta.hip", "permute.hip", "reduce.hip", "allreduce.hip", "scratch.hip"]
HOST_SOURCES = ["abi.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]
# Device code: gfx950 only; packed-fp32 instructions disabled; no fast-math,
# denormals kept (the fixed-order fp32 sums must match IEEE single precision).
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=off"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmd = [cc, *COMMON, *DEVICE, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        jobs.append((src, cmd))
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmd = [cc, *COMMON, "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(CSRC, src), "-o", obj]
        jobs.append((src, cmd))
        objs.append(obj)
    roofline_obj = os.path.join(BUILD, ROOFLINE_SOURCE + ".o")
    jobs.append((ROOFLINE_SOURCE, [cc, *COMMON, *DEVICE, "-x", "hip", "-c", os.path.join(CSRC, ROOFLINE_SOURCE),
                                   "-o", roofline_obj]))
    procs = []
    for src, cmd in jobs:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, cmd, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write(f"--- {src} failed:\n{' '.join(cmd)}\n{text}\n")
        elif verbose and text.strip():
            sys.stderr.write(text)
    if failed:
        raise RuntimeError(f"compilation failed: {failed}")
    tmp = LIB + ".tmp"
    link = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(tmp, LIB)
    tmp = ROOFLINE_LIB + ".tmp"
    r = subprocess.run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", roofline_obj, "-o", tmp],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(tmp, ROOFLINE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
