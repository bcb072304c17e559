"""Build the HIP library in-tree: qk_rope_paged_amd/libqk_rope_paged.so (gfx950).

    python qk_rope_paged_amd/build.py

hipcc compiles the kernels and the C-ABI for gfx950 only.  Packed binary32
instructions are switched off for the device code (-packed-fp32-ops); hipcc's
host pass warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libqk_rope_paged.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["kernels.hip", "kernels_fp8.hip", "kernels_qout.hip", "kernels_pack.hip",
           "kernels_mixed.hip", "gemv_norm.hip", "abi.cpp", "abi_gemv.cpp"]
# measurement helper for the benchmark (not part of the C ABI)
COPY_LIB_PATH = os.path.join(HERE, "libqrp_bench_copy.so")
COPY_SOURCES = ["bench_copy.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-command-line-argument"]


def command(out: str = LIB_PATH, extra=(), sources=SOURCES) -> list:
    """One hipcc line compiling and linking every source (kept for reference
    and for one-off variant builds)."""
    return [hipcc(), *FLAGS, "-shared", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            *[os.path.join(CSRC, s) for s in sources], *extra, "-o", out]


def object_command(src: str, obj: str, extra=()) -> list:
    return [hipcc(), *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c",
            os.path.join(CSRC, src), *extra, "-o", obj]


def _compile(out: str, sources, verbose: bool) -> None:
    """Compile every source to an object in parallel (the kernel translation
    units are independent), then link them into `out`."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in sources]
    procs = [subprocess.Popen(object_command(s, o), stdout=subprocess.PIPE,
                              stderr=subprocess.PIPE, text=True) for s, o in zip(sources, objs)]
    failed = []
    for s, p in zip(sources, procs):
        out_s, err_s = p.communicate()
        if p.returncode != 0:
            failed.append(s)
            sys.stderr.write(out_s + err_s)
        elif verbose:
            sys.stderr.write(err_s)
    if failed:
        raise RuntimeError("hipcc failed on " + ", ".join(failed))
    tmp = out + ".tmp"
    res = subprocess.run([hipcc(), *FLAGS, "-shared", *objs, "-o", tmp], capture_output=True,
                         text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed linking " + os.path.basename(out))
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    _compile(LIB_PATH, SOURCES, verbose)
    _compile(COPY_LIB_PATH, COPY_SOURCES, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
