"""The FP8 and MXFP4 codecs' C ABI without a GPU: buffer sizes as documented, and every
bad argument rejected before anything is launched (fake, aligned, never dereferenced
pointers), as for the KIVI entry points in test_abi_cpu.py."""
import ctypes

import pytest

from tests.test_abi_cpu import FAKE, call

kv = pytest.importorskip("bit_quantization_amd.kivi")


def fp8_dims(**kw):
    d = dict(layers=2, batch=3, kv_heads=2, q_heads=8, head_dim=128, format="e4m3",
             max_tokens=512)
    d.update(kw)
    return kv.Fp8Dims(**d)


def mx_dims(**kw):
    d = dict(layers=2, batch=3, kv_heads=2, q_heads=8, head_dim=128, max_tokens=512)
    d.update(kw)
    return kv.MxDims(**d)


def fake4(cls, **over):
    names = [n for n, _ in cls._fields_]
    ptrs = {n: FAKE + 0x1000000 * i for i, n in enumerate(names)}
    ptrs.update(over)
    return cls(*[ptrs[n] for n in names])


def test_fp8_sizes_follow_the_documented_layout():
    d = fp8_dims()
    unit = d.layers * d.batch * d.kv_heads
    assert kv.kivi_fp8_cache_sizes(d) == [unit * 512 * 128, unit * 512 * 128, 2 * 2 * 4, 2 * 2 * 4]


def test_mxfp4_sizes_follow_the_documented_layout():
    d = mx_dims()
    unit = d.layers * d.batch * d.kv_heads * d.max_tokens
    # k [T][64], k_scale [T][4], v [T/32][128][16], v_scale [T/32][4][32]
    assert kv.kivi_mxfp4_cache_sizes(d) == [unit * 64, unit * 4, unit * 64, unit * 4]


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 64, 2), ("q_heads", 6, 2), ("q_heads", 7, 1), ("max_tokens", 100, 1),
    ("layers", 0, 1), ("reserved", 1, 1),
])
def test_mxfp4_bad_dims_are_rejected(field, value, status):
    c = mx_dims().c()
    setattr(c, field, value)
    sizes = (ctypes.c_size_t * 4)()
    st, msg = call("kivi_mxfp4_cache_sizes", ctypes.byref(c), sizes)
    assert st == status and msg
    st, msg = call("kivi_mxfp4_quantize", ctypes.byref(c), ctypes.byref(fake4(kv.kivi_mxfp4_cache)),
                   0, FAKE, FAKE, 16, 16, None)
    assert st == status and msg


def test_fp8_bad_format_is_rejected():
    c = fp8_dims().c()
    c.format = 7
    st, msg = call("kivi_fp8_quantize", ctypes.byref(c), ctypes.byref(fake4(kv.kivi_fp8_cache)), 0,
                   FAKE, FAKE, 16, 16, None)
    assert st == 2 and "format" in msg


@pytest.mark.parametrize("codec", ["fp8", "mxfp4"])
def test_codec_calls_check_pointers_tokens_and_workspace(codec):
    if codec == "fp8":
        d, cache_cls, pre = fp8_dims().c(), kv.kivi_fp8_cache, "kivi_fp8"
    else:
        d, cache_cls, pre = mx_dims().c(), kv.kivi_mxfp4_cache, "kivi_mxfp4"
    good = fake4(cache_cls)
    first = cache_cls._fields_[0][0]
    # a null or misaligned cache buffer
    st, msg = call(f"{pre}_append", ctypes.byref(d), ctypes.byref(fake4(cache_cls, **{first: None})),
                   0, 3, FAKE, FAKE, None)
    assert st == 1 and first in msg
    st, msg = call(f"{pre}_append", ctypes.byref(d), ctypes.byref(fake4(cache_cls, **{first: FAKE + 4})),
                   0, 3, FAKE, FAKE, None)
    assert st == 4
    # tokens beyond max_tokens, a bad layer
    st, _ = call(f"{pre}_append", ctypes.byref(d), ctypes.byref(good), 0, 512, FAKE, FAKE, None)
    assert st == 3
    st, _ = call(f"{pre}_quantize", ctypes.byref(d), ctypes.byref(good), 0, FAKE, FAKE, 513, 513, None)
    assert st == 3
    st, _ = call(f"{pre}_quantize", ctypes.byref(d), ctypes.byref(good), 2, FAKE, FAKE, 16, 16, None)
    assert st == 1
    # a workspace smaller than the plan's
    need = ctypes.c_size_t()
    assert call(f"{pre}_decode_workspace_bytes", ctypes.byref(d), 500, 0, ctypes.byref(need))[0] == 0
    st, msg = call(f"{pre}_decode_attn", ctypes.byref(d), ctypes.byref(good), 0, 500, FAKE,
                   ctypes.c_float(0.1), FAKE, FAKE, need.value - 1, 0, None)
    assert st == 5 and "workspace" in msg
    st, _ = call(f"{pre}_decode_attn", ctypes.byref(d), ctypes.byref(good), 0, 500, FAKE,
                 ctypes.c_float(float("nan")), FAKE, FAKE, need.value, 0, None)
    assert st == 1


def test_mxfp4_append_decode_checks_before_launching():
    d = mx_dims().c()
    good = fake4(kv.kivi_mxfp4_cache)
    st, _ = call("kivi_mxfp4_append_decode", ctypes.byref(d), ctypes.byref(good), 0, 512, FAKE, FAKE,
                 FAKE, ctypes.c_float(0.1), FAKE, FAKE, 1 << 20, None)
    assert st == 3                       # T_before + 1 = 513 > max_tokens
    st, _ = call("kivi_mxfp4_append_decode", ctypes.byref(d), ctypes.byref(good), 0, 100, None, FAKE,
                 FAKE, ctypes.c_float(0.1), FAKE, FAKE, 1 << 20, None)
    assert st == 1


def test_varlen_lens_pointer_is_checked():
    from tests.test_abi_cpu import fake_cache, good_dims
    d = good_dims().c()
    for lens, status in ((None, 1), (FAKE + 2, 4)):
        st, msg = call("kivi_decode_attn_varlen", ctypes.byref(d), ctypes.byref(fake_cache()), None,
                       0, lens, 16, FAKE, ctypes.c_float(0.1), FAKE, FAKE, 1 << 20, None)
        assert st == status and "lens" in msg


def test_codec_workspaces_never_shrink_as_T_grows():
    """The FP8 and MXFP4 decodes check the workspace against the size for their own T;
    the default split count (capped at one 32-token run per wave) only grows with T,
    so a workspace sized for T serves every smaller T."""
    for dims, size in ((fp8_dims(max_tokens=4096), kv.kivi_fp8_decode_workspace_bytes),
                       (mx_dims(max_tokens=4096), kv.kivi_mxfp4_decode_workspace_bytes)):
        sizes = [size(dims, T) for T in range(1, 3000, 7)]
        assert all(a <= b for a, b in zip(sizes, sizes[1:]))
        assert sizes[-1] > sizes[0]


# FP8 codes take one byte per channel and token, MXFP4 codes half a byte: a pair's
# codes must stay below 2^31 bytes (the kernels' 32-bit buffer offsets).
def test_fp8_capacity_beyond_32bit_offsets_is_unsupported():
    sizes = (ctypes.c_size_t * 4)()
    limit = (1 << 24) - 32
    ok = fp8_dims(max_tokens=limit, layers=1, batch=1, kv_heads=1, q_heads=1).c()
    st, msg = call("kivi_fp8_cache_sizes", ctypes.byref(ok), sizes)
    assert st == 0, msg
    bad = fp8_dims(max_tokens=limit + 32, layers=1, batch=1, kv_heads=1, q_heads=1).c()
    st, msg = call("kivi_fp8_cache_sizes", ctypes.byref(bad), sizes)
    assert st == 2 and "max_tokens" in msg
    st, msg = call("kivi_fp8_quantize", ctypes.byref(bad), ctypes.byref(fake4(kv.kivi_fp8_cache)),
                   0, FAKE, FAKE, 16, 16, None)
    assert st == 2 and "max_tokens" in msg


def test_mxfp4_capacity_beyond_32bit_offsets_is_unsupported():
    sizes = (ctypes.c_size_t * 4)()
    limit = (1 << 25) - 32
    ok = mx_dims(max_tokens=limit, layers=1, batch=1, kv_heads=1, q_heads=1).c()
    st, msg = call("kivi_mxfp4_cache_sizes", ctypes.byref(ok), sizes)
    assert st == 0, msg
    bad = mx_dims(max_tokens=limit + 32, layers=1, batch=1, kv_heads=1, q_heads=1).c()
    st, msg = call("kivi_mxfp4_cache_sizes", ctypes.byref(bad), sizes)
    assert st == 2 and "max_tokens" in msg
    st, msg = call("kivi_mxfp4_quantize", ctypes.byref(bad), ctypes.byref(fake4(kv.kivi_mxfp4_cache)),
                   0, FAKE, FAKE, 16, 16, None)
    assert st == 2 and "max_tokens" in msg
