"""The benchmark's reference-read library without a GPU: it is built apart from
libkivi.so, exports its two entry points, and rejects bad arguments before any launch
(fake, aligned, never dereferenced pointers), and bench.py's pattern shapes are those
of the decode step they stand for."""
import ctypes
import importlib.util
import os

import pytest

import workloads as W
from tests.conftest import ROOT

LIB = os.path.join(ROOT, "bit_quantization_amd", "libkivi_readprobe.so")
FAKE = 0x7F0000000000
P, Z, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libkivi_readprobe.so not built")
    lib = ctypes.CDLL(LIB)
    lib.kivi_probe_pattern_read.restype = I
    lib.kivi_probe_pattern_read.argtypes = [P, Z, I, I, I, I, I, P, Z, P, P, P]
    lib.kivi_probe_stream_read.restype = I
    lib.kivi_probe_stream_read.argtypes = [P, Z, I, I, I, P, Z, P, P, P]
    return lib


def test_entry_points_exported_and_absent_from_the_product(lib):
    assert hasattr(lib, "kivi_probe_pattern_read") and hasattr(lib, "kivi_probe_stream_read")
    product = ctypes.CDLL(os.path.join(ROOT, "bit_quantization_amd", "libkivi.so"))
    assert not hasattr(product, "kivi_probe_pattern_read")
    assert not hasattr(product, "kivi_probe_stream_read")


def pattern(lib, **kw):
    a = dict(buf=FAKE, bytes=64 * 512 * 5376, pairs=64, blocks=512, nw=4, ahead=1, fused=0,
             sink=FAKE, sink_bytes=1 << 22, stream=None, e0=None, e1=None)
    a.update(kw)
    return lib.kivi_probe_pattern_read(a["buf"], a["bytes"], a["pairs"], a["blocks"], a["nw"],
                                       a["ahead"], a["fused"], a["sink"], a["sink_bytes"],
                                       a["stream"], a["e0"], a["e1"])


@pytest.mark.parametrize("kw", [
    dict(buf=None), dict(buf=FAKE + 8), dict(sink=None), dict(pairs=0), dict(blocks=0),
    dict(nw=0), dict(nw=513), dict(ahead=0), dict(ahead=4), dict(bytes=64 * 512 * 5376 - 1),
    dict(sink_bytes=64 * 4 * 512 * 4 - 1), dict(blocks=1 << 19, bytes=1 << 40),
    dict(pairs=65537, nw=1, bytes=1 << 40), dict(e0=FAKE),
])
def test_pattern_read_rejects_bad_arguments(lib, kw):
    assert pattern(lib, **kw) == 1


def test_pattern_shapes_are_the_decode_steps():
    spec = importlib.util.spec_from_file_location("bench_rp", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    for name, pairs, blocks, nw in bench.PATTERN_SHAPES:
        w = W.get(name)
        assert w.bits == 2 and w.group_k == 32 and w.head_dim == 128
        assert pairs == w.batch * w.kv_heads
        # the quantized history's whole 64-token blocks (the window holds the rest)
        assert blocks == (w.tokens - w.residual) // 64
        assert nw == 256 // pairs
