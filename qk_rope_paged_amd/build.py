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
SOURCES = ["kernels.hip", "abi.cpp"]
# measurement helper for the benchmark (not part of the C ABI)
COPY_LIB_PATH = os.path.join(HERE, "libqrp_bench_copy.so")
COPY_SOURCES = ["bench_copy.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def command(out: str = LIB_PATH, extra=(), sources=SOURCES) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            *[os.path.join(CSRC, s) for s in sources], *extra, "-o", out]


def _compile(out: str, sources, verbose: bool) -> None:
    tmp = out + ".tmp"
    res = subprocess.run(command(tmp, sources=sources), capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building " + os.path.basename(out))
    if verbose:
        sys.stderr.write(res.stderr)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    _compile(LIB_PATH, SOURCES, verbose)
    _compile(COPY_LIB_PATH, COPY_SOURCES, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
