"""kivi_time_next_decode: the armed decode launch records the caller's two events at the
decode kernel's own start and end (the measurement aid the benchmark's roofline uses).

Checks: the recorded duration is positive and within the step's own event bracket, the
output is the same as without the timer (within the stated tolerance of the oracle), only
the next decode launch is timed, and the FP8 and MXFP4 decodes honour it too."""
import math

import numpy as np
import pytest

import oracle as O
import workloads as W
from tests.test_gpu_parity import assert_close, gpu_prefill, rand_kv

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def kv():
    from bit_quantization_amd import kivi
    return kivi


def events(n):
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in ev:
        e.record(stream)
    torch.cuda.synchronize()
    return ev


def test_kernel_clock_times_the_decode_kernel():
    k = kv()
    B, H, g, T, d = 2, 2, 4, 3000, 128
    print("[clock] kivi decode", flush=True)
    w = W.Workload("clk", 97, 1, B, H, H * g, d, T, 2, 32, d, 128)
    m = math.lcm(16, 32, 128)
    dims = k.Dims(layers=1, batch=B, kv_heads=H, q_heads=H * g, head_dim=d, bits=2, group_k=32,
                  group_v=d, residual=128, max_tokens=(T + 64 + m) // m * m)
    K, V = rand_kv(B, H, T, d, seed=3)
    cache = gpu_prefill(w, dims, K, V, T)
    q = torch.randn((B, H * g, d), device="cuda").to(torch.float16)
    ws = k.new_workspace(dims, T)
    out = torch.empty((B, H * g, d), dtype=torch.float32, device="cuda")
    ks, kt, s0, s1 = events(4)
    stream = torch.cuda.current_stream()
    s0.record(stream)
    k.kivi_time_next_decode(ks.cuda_event, kt.cuda_event)
    k.kivi_decode_attn(dims, cache, 0, T, q, 0.09, out, ws)
    s1.record(stream)
    torch.cuda.synchronize()
    kernel_ms, step_ms = ks.elapsed_time(kt), s0.elapsed_time(s1)
    assert 0 < kernel_ms <= step_ms, (kernel_ms, step_ms)
    oc = O.LayerCache(B, H, d, 2, 32, d, 128, dims.max_tokens)
    oc.prefill(K.cpu().numpy(), V.cpu().numpy())
    assert_close(out.cpu().numpy(), oc.attend(q.cpu().numpy(), 0.09), "timed decode")
    # the timer was taken by that launch: the next one leaves the events alone
    k.kivi_decode_attn(dims, cache, 0, T, q, 0.09, out, ws)
    torch.cuda.synchronize()
    assert ks.elapsed_time(kt) == kernel_ms


@pytest.mark.parametrize("codec", ["fp8", "mxfp4"])
def test_kernel_clock_codecs(codec):
    k = kv()
    B, H, g, T, d = 1, 2, 4, 2000, 128
    print(f"[clock] {codec} decode", flush=True)
    K, V = rand_kv(B, H, T, d, seed=4)
    q = torch.randn((B, H * g, d), device="cuda").to(torch.float16)
    out = torch.empty((B, H * g, d), dtype=torch.float32, device="cuda")
    if codec == "fp8":
        dims = k.Fp8Dims(layers=1, batch=B, kv_heads=H, q_heads=H * g, head_dim=d,
                         format="e4m3", max_tokens=2112)
        cache = k.Fp8Cache(dims)
        k.kivi_fp8_quantize(dims, cache, 0, K, V, T, K.shape[2])
        ws = k.new_fp8_workspace(dims, T)
        run = lambda: k.kivi_fp8_decode_attn(dims, cache, 0, T, q, 0.09, out, ws)
    else:
        dims = k.MxDims(layers=1, batch=B, kv_heads=H, q_heads=H * g, head_dim=d,
                        max_tokens=2112)
        cache = k.MxCache(dims)
        k.kivi_mxfp4_quantize(dims, cache, 0, K, V, T, K.shape[2])
        ws = k.new_mxfp4_workspace(dims, T)
        run = lambda: k.kivi_mxfp4_decode_attn(dims, cache, 0, T, q, 0.09, out, ws)
    ks, kt, s0, s1 = events(4)
    stream = torch.cuda.current_stream()
    s0.record(stream)
    k.kivi_time_next_decode(ks.cuda_event, kt.cuda_event)
    run()
    s1.record(stream)
    torch.cuda.synchronize()
    kernel_ms, step_ms = ks.elapsed_time(kt), s0.elapsed_time(s1)
    assert 0 < kernel_ms <= step_ms, (kernel_ms, step_ms)
