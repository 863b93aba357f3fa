"""The library's host code (argument validation, planning, the C ABI) built with
AddressSanitizer and UndefinedBehaviorSanitizer, and the CPU ABI tests run against that
build (no GPU: every call stops at its checks or at the first HIP call).  Kernels are
compiled as in the product build; only the host side is instrumented."""
import glob
import hashlib
import os
import subprocess
import sys

import pytest

from tests.conftest import ROOT

BUILD = os.path.join(ROOT, "tests", "c", "_build")
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
            "-fno-omit-frame-pointer"]


def load_build_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "kivi_build", os.path.join(ROOT, "bit_quantization_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def asan_runtime():
    libs = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return libs[-1] if libs else None


def sanitized_library():
    B = load_build_module()
    srcs = [os.path.join(B.CSRC, n) for n in B.SOURCES]
    h = hashlib.sha256()
    for path in srcs + sorted(glob.glob(os.path.join(B.CSRC, "*.h"))) + [
            os.path.join(B.INCLUDE, "kivi.h")]:
        h.update(open(path, "rb").read())
    os.makedirs(BUILD, exist_ok=True)
    lib = os.path.join(BUILD, f"libkivi_hostsan_{h.hexdigest()[:16]}.so")
    if os.path.exists(lib):
        return lib
    flags = [f for f in B.HIPCC_FLAGS if f != "-shared"]
    objs, procs = [], []
    for src in srcs:
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        objs.append(obj)
        procs.append(subprocess.Popen(
            [B.hipcc(), *flags, *SANITIZE, "-c", "-I", B.INCLUDE, "-I", B.CSRC, "-x", "hip", src,
             "-o", obj], stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
    for p in procs:
        out = p.communicate()[0]
        assert p.returncode == 0, out.decode()[-2000:]
    subprocess.run([B.hipcc(), "--offload-arch=gfx950", "-shared", *SANITIZE, *objs, "-o", lib],
                   check=True, capture_output=True)
    return lib


@pytest.mark.skipif(asan_runtime() is None, reason="no AddressSanitizer runtime in this toolchain")
def test_abi_checks_under_host_sanitizers():
    lib = sanitized_library()
    # the host code is instrumented: the library calls the sanitizer runtimes
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan_runtime(), KIVI_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          "-m", "not gpu", "tests/test_abi_cpu.py", "tests/test_abi_codecs_cpu.py"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
