"""The C ABI without a GPU: the library loads, exports what include/kivi.h declares,
sizes buffers as documented, and rejects every bad argument before launching.

No test here ever reaches a launch: each call fails validation first, so fake
(aligned, never dereferenced) pointers are safe.
"""
import ctypes
import os
import re
import subprocess

import pytest
import torch

from tests.conftest import ROOT

kv = pytest.importorskip("bit_quantization_amd.kivi")

HEADER = os.path.join(ROOT, "include", "kivi.h")
FAKE = 0x7F0000000000          # 16-byte aligned, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:kivi_status|const char\*|int32_t)\s+(kivi_\w+)\s*\(",
                                 text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"kivi_quantize_k", "kivi_quantize_v", "kivi_append_flush",
            "kivi_decode_attn"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", kv.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (kivi_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert set(kv.EXPORTS) == set(names)


def test_abi_version():
    assert kv.kivi_abi_version() == 9


def good_dims(**kw):
    d = dict(layers=2, batch=3, kv_heads=2, q_heads=8, head_dim=128, bits=2, group_k=32,
             group_v=128, residual=64, max_tokens=512)
    d.update(kw)
    return kv.Dims(**d)


def fake_cache(**overrides):
    ptrs = {n: FAKE + 0x1000000 * i for i, n in enumerate(kv.BUFFERS)}
    ptrs.update(overrides)
    return kv.kivi_cache(*[ptrs[n] for n in kv.BUFFERS])


def call(fn, *args):
    st = getattr(kv._lib, fn)(*args)
    return st, kv._lib.kivi_last_error().decode()


def test_cache_sizes_follow_the_documented_layout():
    d = good_dims(bits=4, group_v=64)
    sizes = kv.kivi_cache_sizes(d)
    unit = d.layers * d.batch * d.kv_heads
    codes = unit * d.max_tokens * d.head_dim * d.bits // 8
    assert sizes == [codes, unit * (d.max_tokens // 32) * 128 * 2, unit * (d.max_tokens // 32) * 128 * 2,
                     codes, unit * d.max_tokens * 2 * 2, unit * d.max_tokens * 2 * 2,
                     unit * 64 * 128 * 2, unit * 64 * 128 * 2, unit * 2 * 4]


@pytest.mark.parametrize("field,value,status", [
    ("bits", 3, 2), ("bits", 8, 2), ("head_dim", 64, 2), ("group_k", 48, 2),
    ("group_v", 48, 1), ("group_v", 8, 2), ("residual", 40, 1), ("residual", 0, 1),
    ("q_heads", 7, 1), ("q_heads", 32, 2), ("max_tokens", 100, 1), ("layers", 0, 1),
    ("batch", 0, 1), ("kv_heads", 0, 1),
])
def test_bad_dims_are_rejected(field, value, status):
    d = good_dims(**{field: value})
    sizes = (ctypes.c_size_t * len(kv.BUFFERS))()
    st, msg = call("kivi_cache_sizes", ctypes.byref(d.c()), sizes)
    assert st == status and msg
    st, msg = call("kivi_quantize_k", ctypes.byref(d.c()), ctypes.byref(fake_cache()), 0, FAKE,
                   16, 16, None)
    assert st == status and msg


@pytest.mark.parametrize("sink", [-1, 1025])
def test_sink_out_of_range_is_rejected(sink):
    c = good_dims().c()
    c.sink = sink
    st, msg = call("kivi_quantize_v", ctypes.byref(c), ctypes.byref(fake_cache()), 0, FAKE, 16, 16,
                   None)
    assert st == 1 and "sink" in msg


def test_sink_rows_extend_the_float16_buffers():
    d = good_dims(bits=4, group_v=64)
    d.sink = 7
    sizes = kv.kivi_cache_sizes(d)
    unit = d.layers * d.batch * d.kv_heads
    assert sizes[6] == sizes[7] == unit * (7 + 64) * 128 * 2
    d.sink = 0
    assert kv.kivi_cache_sizes(d)[6] == unit * 64 * 128 * 2


def test_null_and_misaligned_pointers():
    d = good_dims().c()
    st, msg = call("kivi_quantize_k", ctypes.byref(d), ctypes.byref(fake_cache(k_scale=0)), 0,
                   FAKE, 16, 16, None)
    assert st == 1 and "k_scale" in msg
    st, msg = call("kivi_quantize_k", ctypes.byref(d), ctypes.byref(fake_cache(scale_max=0)), 0,
                   FAKE, 16, 16, None)
    assert st == 1 and "scale_max" in msg
    st, msg = call("kivi_quantize_k", ctypes.byref(d), ctypes.byref(fake_cache(v_resid=FAKE + 8)),
                   0, FAKE, 16, 16, None)
    assert st == 4 and "v_resid" in msg
    st, _ = call("kivi_quantize_k", ctypes.byref(d), ctypes.byref(fake_cache()), 0, None, 16, 16,
                 None)
    assert st == 1
    st, _ = call("kivi_quantize_k", ctypes.byref(d), ctypes.byref(fake_cache()), 0, FAKE + 2, 16,
                 16, None)
    assert st == 4
    st, _ = call("kivi_append_flush", ctypes.byref(d), ctypes.byref(fake_cache()), 0, 5, FAKE,
                 FAKE + 4, None)
    assert st == 4
    st, _ = call("kivi_cache_sizes", None, (ctypes.c_size_t * len(kv.BUFFERS))())
    assert st == 1
    st, _ = call("kivi_quantize_k", ctypes.byref(d), None, 0, FAKE, 16, 16, None)
    assert st == 1


def test_layer_token_and_capacity_checks():
    d = good_dims().c()
    c = ctypes.byref(fake_cache())
    assert call("kivi_quantize_k", ctypes.byref(d), c, 2, FAKE, 16, 16, None)[0] == 1
    assert call("kivi_quantize_k", ctypes.byref(d), c, -1, FAKE, 16, 16, None)[0] == 1
    assert call("kivi_quantize_k", ctypes.byref(d), c, 0, FAKE, 513, 513, None)[0] == 3
    assert call("kivi_quantize_k", ctypes.byref(d), c, 0, FAKE, 16, 8, None)[0] == 1
    assert call("kivi_quantize_k", ctypes.byref(d), c, 0, FAKE, -1, 0, None)[0] == 1
    assert call("kivi_append_flush", ctypes.byref(d), c, 0, 512, FAKE, FAKE, None)[0] == 3
    assert call("kivi_append_flush", ctypes.byref(d), c, 0, -1, FAKE, FAKE, None)[0] == 1
    # T == 0 quantizes nothing and succeeds without touching the GPU
    assert call("kivi_quantize_k", ctypes.byref(d), c, 0, None, 0, 0, None)[0] == 0


def test_decode_argument_checks():
    d = good_dims()
    dc = d.c()
    c = ctypes.byref(fake_cache())
    need = kv.kivi_decode_workspace_bytes(d, 300)
    assert need > 0
    args = lambda T, q, out, ws, wsb: (ctypes.byref(dc), c, 0, T, q, ctypes.c_float(0.1), out,
                                       ws, wsb, None)
    assert call("kivi_decode_attn", *args(0, FAKE, FAKE, FAKE, need))[0] == 1
    assert call("kivi_decode_attn", *args(513, FAKE, FAKE, FAKE, need))[0] == 3
    assert call("kivi_decode_attn", *args(300, None, FAKE, FAKE, need))[0] == 1
    assert call("kivi_decode_attn", *args(300, FAKE, FAKE + 4, FAKE, need))[0] == 4
    assert call("kivi_decode_attn", *args(300, FAKE, FAKE, None, need))[0] == 5
    assert call("kivi_decode_attn", *args(300, FAKE, FAKE, FAKE, need - 1))[0] == 5
    bad = ctypes.byref(dc), c, 0, 300, FAKE, ctypes.c_float(float("nan")), FAKE, FAKE, need, None
    assert call("kivi_decode_attn", *bad)[0] == 1
    # decode kernels need G_v == d and G in {32, 64}
    d2 = good_dims(group_v=64).c()
    assert call("kivi_decode_attn", ctypes.byref(d2), c, 0, 300, FAKE, ctypes.c_float(0.1), FAKE,
                FAKE, need, None)[0] == 2
    d3 = good_dims(group_k=16).c()
    assert call("kivi_decode_attn", ctypes.byref(d3), c, 0, 300, FAKE, ctypes.c_float(0.1), FAKE,
                FAKE, need, None)[0] == 2


def test_append_decode_argument_checks():
    d = good_dims()
    dc = d.c()
    c = ctypes.byref(fake_cache())
    need = kv.kivi_decode_workspace_bytes(d, 301)
    args = lambda Tb, kn, vn, q, out, ws, wsb: (ctypes.byref(dc), c, 0, Tb, kn, vn, q,
                                               ctypes.c_float(0.1), out, ws, wsb, None)
    assert call("kivi_append_decode", *args(512, FAKE, FAKE, FAKE, FAKE, FAKE, need))[0] == 3
    assert call("kivi_append_decode", *args(-1, FAKE, FAKE, FAKE, FAKE, FAKE, need))[0] == 1
    assert call("kivi_append_decode", *args(300, None, FAKE, FAKE, FAKE, FAKE, need))[0] == 1
    assert call("kivi_append_decode", *args(300, FAKE, FAKE + 4, FAKE, FAKE, FAKE, need))[0] == 4
    assert call("kivi_append_decode", *args(300, FAKE, FAKE, None, FAKE, FAKE, need))[0] == 1
    assert call("kivi_append_decode", *args(300, FAKE, FAKE, FAKE, FAKE + 8, FAKE, need))[0] == 4
    assert call("kivi_append_decode", *args(300, FAKE, FAKE, FAKE, FAKE, None, need))[0] == 5
    # the workspace is sized for T_before + 1 tokens
    assert call("kivi_append_decode", *args(300, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1))[0] == 5
    st, msg = call("kivi_append_decode", ctypes.byref(dc), ctypes.byref(fake_cache(v_resid=0)), 0,
                   300, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE, FAKE, need, None)
    assert st == 1 and "v_resid" in msg


def test_split_plan_is_clamped_and_workspace_grows_with_splits():
    d = good_dims()
    # one workgroup per (sequence, KV head) takes the fp16 window, the others split the
    # 64-token blocks of the quantized history (R = 64 here): at most 1 + blocks
    most = lambda T: 1 + (T - ((T - 1) % 64 + 1) + 63) // 64
    assert most(300) == 1 + 4
    assert 1 <= kv.kivi_decode_splits(d, 300) <= most(300)
    assert kv.kivi_decode_splits(d, 10) == 1          # nothing quantized yet: the window
    a = kv.kivi_decode_workspace_bytes(d, 448, 1)
    b = kv.kivi_decode_workspace_bytes(d, 448, 4)
    assert b > a
    assert most(448) == 1 + 6
    assert kv.kivi_decode_workspace_bytes(d, 448, 1000) == kv.kivi_decode_workspace_bytes(d, 448, 7)
    assert kv.kivi_decode_workspace_bytes(d, 448, 7) > kv.kivi_decode_workspace_bytes(d, 448, 6)


@pytest.mark.parametrize("field,value", [("aging", 2), ("aging", -1), ("flags", 4), ("flags", -8)])
def test_aging_and_flags_fields_are_checked(field, value):
    c = good_dims().c()
    setattr(c, field, value)
    st, msg = call("kivi_quantize_k", ctypes.byref(c), ctypes.byref(fake_cache()), 0, FAKE, 16, 16,
                   None)
    assert st == 1 and field in msg


def test_paged_cache_sizes_follow_the_documented_layout():
    d = good_dims(bits=4, group_v=64)
    pg = kv.Paging(page_tokens=128, pages_per_seq=d.max_tokens // 128 + 1, pages=37)
    sizes = kv.kivi_paged_cache_sizes(d, pg)
    sec = d.layers * d.kv_heads
    unit = d.layers * d.batch * d.kv_heads
    rows = 37 * 128
    codes = sec * rows * d.head_dim * d.bits // 8
    assert sizes == [codes, sec * (rows // 32) * 128 * 2, sec * (rows // 32) * 128 * 2,
                     codes, sec * rows * 2 * 2, sec * rows * 2 * 2,
                     unit * 64 * 128 * 2, unit * 64 * 128 * 2, unit * 2 * 4]


@pytest.mark.parametrize("P,per_seq,pages,status", [
    (100, 64, 8, 1), (32, 64, 8, 1), (128, 64, 0, 1), (128, 0, 8, 1),
    (128, 1, 8, 3),                       # 128 tokens per sequence < max_tokens
    (1 << 20, 1, 1 << 12, 2),             # a head's pool beyond 2^31 bytes
])
def test_bad_paging_is_rejected(P, per_seq, pages, status):
    d = good_dims()
    pg = kv.kivi_paging(P, per_seq, pages, FAKE)
    sizes = (ctypes.c_size_t * len(kv.BUFFERS))()
    st, msg = call("kivi_paged_cache_sizes", ctypes.byref(d.c()), ctypes.byref(pg), sizes)
    assert st == status and msg
    lens = FAKE
    st, msg = call("kivi_quantize_k_varlen", ctypes.byref(d.c()), ctypes.byref(fake_cache()),
                   ctypes.byref(pg), 0, FAKE, lens, 16, 16, None)
    assert st == status and msg


def test_paged_calls_check_the_block_table_pointer():
    d = good_dims()
    for table, status in ((None, 1), (FAKE + 2, 4)):
        pg = kv.kivi_paging(128, d.max_tokens // 128 + 1, 8, table)
        st, msg = call("kivi_decode_attn_varlen", ctypes.byref(d.c()), ctypes.byref(fake_cache()),
                       ctypes.byref(pg), 0, FAKE, 16, FAKE, ctypes.c_float(0.1), FAKE, FAKE,
                       1 << 20, None)
        assert st == status and "block_table" in msg


def test_default_split_keeps_every_wave_busy():
    """The default split count is one workgroup per CU (256 / pairs) unless the pair's
    work (64-token blocks, float16 chunks counted as 3 blocks) would leave some of a
    workgroup's waves (12 at g <= 2 and 2 bits, 8 at g = 4) without an item."""
    big = dict(layers=1, max_tokens=140000, head_dim=128, bits=2, group_k=32, group_v=128,
               residual=128)
    d = kv.Dims(batch=8, kv_heads=8, q_heads=32, **big)          # 64 pairs, 8 waves
    assert kv.kivi_decode_splits(d, 32769) == 4                   # 256 / 64
    # T = 300: 256 quantized tokens (4 blocks) + 44 float16 rows (2 chunks) = 10 items
    assert kv.kivi_decode_splits(d, 300) == 2
    d = kv.Dims(batch=1, kv_heads=1, q_heads=1, **big)            # 1 pair, 12 waves
    # T = 257: 4 blocks + one chunk = 7 items: one workgroup, no merge
    assert kv.kivi_decode_splits(d, 257) == 1
    # T = 131073: 2048 blocks + one chunk = 2051 items -> 171 workgroups of 12 waves
    assert kv.kivi_decode_splits(d, 131073) == 171
    d = kv.Dims(batch=1, kv_heads=8, q_heads=32, **big)           # 8 pairs
    assert kv.kivi_decode_splits(d, 131073) == 32                 # 256 / 8


def test_workspace_for_T_serves_every_smaller_T():
    """kivi_decode_attn checks the workspace against the size for its own T: the size
    must never fall as T grows (across flushes the default split count does)."""
    for g, bits in ((4, 2), (2, 4), (8, 2)):
        d = kv.Dims(layers=1, batch=2, kv_heads=2, q_heads=2 * g, head_dim=128, bits=bits,
                    group_k=32, group_v=128, residual=128, max_tokens=4096)
        sizes = [kv.kivi_decode_workspace_bytes(d, T) for T in range(1, 1400)]
        assert all(a <= b for a, b in zip(sizes, sizes[1:]))
        splits = [kv.kivi_decode_splits(d, T) for T in range(1, 1400)]
        assert any(a > b for a, b in zip(splits, splits[1:]))   # the count itself does fall


# The kernels address one (sequence, KV head) pair's history with 32-bit buffer offsets,
# so a pair's codes (its largest buffer: d*b/8 bytes per token) must stay below 2^31
# bytes: at 2 bits the largest capacity is the last multiple of 32 tokens under 2^26, at
# 4 bits under 2^25.
@pytest.mark.parametrize("bits,limit", [(2, (1 << 26) - 32), (4, (1 << 25) - 32)])
def test_capacity_beyond_32bit_offsets_is_unsupported(bits, limit):
    sizes = (ctypes.c_size_t * len(kv.BUFFERS))()
    ok = good_dims(bits=bits, max_tokens=limit, layers=1, batch=1, kv_heads=1, q_heads=1)
    st, msg = call("kivi_cache_sizes", ctypes.byref(ok.c()), sizes)
    assert st == 0, msg
    assert sizes[0] < (1 << 31)
    bad = good_dims(bits=bits, max_tokens=limit + 32, layers=1, batch=1, kv_heads=1, q_heads=1)
    st, msg = call("kivi_cache_sizes", ctypes.byref(bad.c()), sizes)
    assert st == 2 and "max_tokens" in msg
    # every entry point that takes the dims rejects it before launching
    st, msg = call("kivi_quantize_k", ctypes.byref(bad.c()), ctypes.byref(fake_cache()), 0, FAKE,
                   16, 16, None)
    assert st == 2 and "max_tokens" in msg
    need = ctypes.c_size_t(0)
    st, msg = call("kivi_decode_workspace_bytes", ctypes.byref(bad.c()), 300, ctypes.byref(need))
    assert st == 2


def test_noalloc_step_rejects_scratch_beyond_its_maximum():
    # 32768 (sequence, KV head) pairs need 8 MiB of arrival counters alone, more than the
    # 4 MiB static scratch: rejected before anything is enqueued (fake pointers, no GPU)
    d = good_dims(layers=1, batch=128, kv_heads=256, q_heads=1024, max_tokens=512)
    st, msg = call("kivi_append_decode_noalloc", ctypes.byref(d.c()), ctypes.byref(fake_cache()),
                   0, 300, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE, None)
    assert st == 2 and "scratch" in msg, msg
    # argument checks come first, as for kivi_append_decode
    st, msg = call("kivi_append_decode_noalloc", ctypes.byref(good_dims().c()),
                   ctypes.byref(fake_cache()), 0, 512, FAKE, FAKE, FAKE, ctypes.c_float(0.1),
                   FAKE, None)
    assert st == 3, msg
    st, msg = call("kivi_append_decode_noalloc", ctypes.byref(good_dims().c()),
                   ctypes.byref(fake_cache()), 0, 300, None, FAKE, FAKE, ctypes.c_float(0.1),
                   FAKE, None)
    assert st == 1, msg


def test_value_token_window_is_refused_for_ragged_and_paged_calls():
    # KIVI_FLAG_VALUE_TOKEN_WINDOW is built for uniform batches in contiguous caches: the
    # ragged and paged entry points refuse it before launching (fake pointers, no GPU)
    d = good_dims(v_window="token")
    pg = kv.kivi_paging(128, d.max_tokens // 128 + 1, 37, FAKE)
    st, msg = call("kivi_quantize_k_varlen", ctypes.byref(d.c()), ctypes.byref(fake_cache()),
                   ctypes.byref(pg), 0, FAKE, FAKE, 300, 300, None)
    assert st == 2 and "VALUE_TOKEN_WINDOW" in msg, msg
    st, msg = call("kivi_append_flush_varlen", ctypes.byref(d.c()), ctypes.byref(fake_cache()),
                   None, 0, FAKE, 300, FAKE, FAKE, None)
    assert st == 2 and "VALUE_TOKEN_WINDOW" in msg, msg
    need = ctypes.c_size_t(1 << 20)
    st, msg = call("kivi_append_decode_varlen", ctypes.byref(d.c()), ctypes.byref(fake_cache()),
                   None, 0, FAKE, 300, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE, FAKE,
                   need, None)
    assert st == 2 and "VALUE_TOKEN_WINDOW" in msg, msg
    # the uniform calls accept it (sizes are the same as without it)
    assert kv.kivi_cache_sizes(d) == kv.kivi_cache_sizes(good_dims())


def test_time_next_decode_arguments():
    # host-only: the measurement aid takes both events or neither, and launches nothing
    with pytest.raises(kv.KiviError, match="ARG"):
        kv.kivi_time_next_decode(1, None)
    with pytest.raises(kv.KiviError, match="ARG"):
        kv.kivi_time_next_decode(None, 1)
    kv.kivi_time_next_decode()


def test_host_length_step_checks_its_host_copy():
    # kivi_append_decode_varlen_host refuses a missing host copy and entries outside
    # [0, T_hi] before it launches anything (fake device pointers, no GPU)
    d = good_dims()
    need = kv.kivi_decode_workspace_bytes(d, 301)
    args = lambda host: (ctypes.byref(d.c()), ctypes.byref(fake_cache()), None, 0, FAKE, host,
                         300, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE, FAKE, need, None)
    st, msg = call("kivi_append_decode_varlen_host", *args(None))
    assert st == 1 and "T_before_host" in msg, msg
    for bad in ((0, 5, -1), (0, 301, 7)):
        host = (ctypes.c_int32 * d.batch)(*bad)
        st, msg = call("kivi_append_decode_varlen_host", *args(host))
        assert st == 1 and "T_before_host" in msg, msg
    # the checks shared with kivi_append_decode_varlen come first
    host = (ctypes.c_int32 * d.batch)(0, 1, 2)
    st, msg = call("kivi_append_decode_varlen_host", *args(host)[:4], None, host,
                   *args(host)[6:])
    assert st == 1 and "lens" in msg, msg
    dw = good_dims(v_window="token")
    st, msg = call("kivi_append_decode_varlen_host", ctypes.byref(dw.c()),
                   *args(host)[1:])
    assert st == 2 and "VALUE_TOKEN_WINDOW" in msg, msg


def test_host_length_binding_takes_a_cpu_int32_tensor():
    d = good_dims()
    with pytest.raises(ValueError, match="CPU"):
        kv._host_lens(torch.zeros(3, dtype=torch.int64), d)
    with pytest.raises(ValueError, match="needs 3"):
        kv._host_lens(torch.zeros(2, dtype=torch.int32), d)
    with pytest.raises(TypeError):
        kv._host_lens([0, 1, 2], d)
    t = torch.zeros(3, dtype=torch.int32)
    assert kv._host_lens(t, d) == t.data_ptr()
