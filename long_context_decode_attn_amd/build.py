"""Build libuocr.so (gfx950) in-tree with hipcc.

    python -m long_context_decode_attn_amd.build

compiles csrc/uocr_kernels.hip, csrc/uocr_api.cpp and csrc/uocr_calib.hip into
long_context_decode_attn_amd/libuocr.so, and the same sources with the
kernels' phase stamps compiled in (UOCR_PHASE_STAMPS) into
libuocr_stamps.so, the library `bench.py --phases` measures with.  Packed
fp32 instructions are switched off for all device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libuocr.so")
STAMPS_LIB = os.path.join(HERE, "libuocr_stamps.so")
SOURCES = [os.path.join(CSRC, "uocr_kernels.hip"), os.path.join(CSRC, "uocr_api.cpp"),
           os.path.join(CSRC, "uocr_calib.hip")]

ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libuocr.so)")


def compile_flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        "-Wno-unused-function",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        "-I", CSRC,
    ]


def build_library(verbose: bool = True) -> str:
    """Compile every source to an object, link libuocr.so and
    libuocr_stamps.so, return the path of libuocr.so."""
    cc = hipcc()
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    jobs = []   # (source, object, extra flags)
    for src in SOURCES:
        jobs.append((src, os.path.join(objdir, os.path.basename(src) + ".o"), []))
    kernels = SOURCES[0]
    jobs.append((kernels, os.path.join(objdir, "stamps_" + os.path.basename(kernels) + ".o"),
                 ["-DUOCR_PHASE_STAMPS"]))
    procs = []
    for src, obj, extra in jobs:   # the sources compile in parallel
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [cc, *compile_flags(), *extra, *lang, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd)))
    for cmd, p in procs:
        if p.wait() != 0:
            raise subprocess.CalledProcessError(p.returncode, cmd)
    plain = [obj for _, obj, extra in jobs if not extra]
    stamped = [jobs[-1][1]] + plain[1:]
    for out, objs in ((LIB, plain), (STAMPS_LIB, stamped)):
        tmp = out + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return LIB


if __name__ == "__main__":
    build_library(verbose="-q" not in sys.argv)
    print(LIB)
