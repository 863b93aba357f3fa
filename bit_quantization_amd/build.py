"""Build the HIP libraries in-tree for gfx950 with hipcc.

``libkivi.so``: the sources listed in SOURCES (the C ABI and its kernels).
``libkivi_readprobe.so``: the reference reads the benchmark compares the decode with, a
plain streaming read and the decode's access pattern without its arithmetic
(``csrc/bench/``); not part of the method and not loaded by the package.
``libkivi_timeline.so``: libkivi.so's sources built with KIVI_TIMELINE, whose decode
kernel stamps per-workgroup clocks (``bench.py --timeline``); never the product.
Run as ``python bit_quantization_amd/build.py`` (by path: importing the package loads
the library it builds).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libkivi.so")
PROBE_LIB = os.path.join(HERE, "libkivi_readprobe.so")
TIMELINE_LIB = os.path.join(HERE, "libkivi_timeline.so")

SOURCES = ["kivi_api.cpp", "quantize.hip", "decode.hip", "fp8.hip", "mxfp4.hip"]
PROBE_SOURCES = [os.path.join("bench", "read_probe.hip")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep packed float32 instructions out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE float32 division/sqrt (the quantizer's arithmetic is bit-exact by contract)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall",
    "-Wno-unused-function",
    # a kernel that misses the occupancy its launch bounds ask for is a build error:
    # the split planner sizes the grid from that occupancy
    "-Werror=pass-failed",
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the HIP toolchain is required to build libkivi.so")
    return exe


def _build(sources, lib, verbose, defines=()):
    srcs = []
    for name in sources:
        # every source compiles as HIP (the API file includes the HIP runtime headers)
        srcs += ["-x", "hip", os.path.join(CSRC, name)]
    tmp = lib + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *["-D" + d for d in defines], "-I", INCLUDE, "-I", CSRC,
           *srcs, "-o", tmp]
    if verbose:
        print("[build]", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


def build_library(verbose: bool = True) -> str:
    """Build libkivi.so and the benchmark's read-probe and timeline libraries; returns
    libkivi.so's path."""
    _build(PROBE_SOURCES, PROBE_LIB, verbose)
    _build(SOURCES, TIMELINE_LIB, verbose, defines=("KIVI_TIMELINE=1",))
    return _build(SOURCES, LIB, verbose)


if __name__ == "__main__":
    build_library()
    sys.exit(0)
