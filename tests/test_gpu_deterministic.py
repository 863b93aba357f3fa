"""KIVI_FLAG_DETERMINISTIC: repeated decode calls give the same output bits.

With the flag every wave of a workgroup takes a fixed round-robin share of the 64-token
blocks (window chunks weighted as three blocks), so the float sums a wave forms and the
order of the fixed-order merge no longer depend on the run.  Each case repeats the call
and compares the bits, and checks the first result against the oracle (the stated
tolerance |gpu - ref| <= 2e-3 + 1e-3 |ref|).
"""
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


def det_dims(w, S=0, aging="window"):
    m = math.lcm(16, w.group_k, w.residual)
    Tmax = (w.max_tokens() + S + 64 + m - 1) // m * m
    return kv().Dims(layers=w.layers, batch=w.batch, kv_heads=w.kv_heads, q_heads=w.q_heads,
                     head_dim=w.head_dim, bits=w.bits, group_k=w.group_k, group_v=w.group_v,
                     residual=w.residual, max_tokens=Tmax, sink=S, aging=aging,
                     deterministic=True)


def bits_of(t):
    return t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("bits,G,R,B,H,g,T,S,n_split", [
    (2, 32, 128, 2, 2, 4, 5000, 0, 0),
    (2, 32, 128, 2, 2, 4, 5000, 0, 3),
    (4, 64, 64, 1, 3, 8, 2117, 0, 0),      # 8 query heads per KV head
    (2, 32, 32, 3, 1, 2, 999, 0, 5),       # a 32-token last block
    (2, 32, 128, 1, 2, 4, 3100, 1024, 0),  # 1024 sink rows: 36 window chunks over 8 waves
    (4, 32, 64, 1, 1, 1, 70, 6, 0),        # a few blocks, window-heavy
    (2, 32, 64, 1, 2, 4, 5000, 0, 40),     # a merge of 40 partials in two rounds
    (4, 64, 64, 1, 1, 8, 3000, 0, 37),     # 8 query heads: three rounds of up to 16
])
def test_deterministic_decode_repeats_bits(bits, G, R, B, H, g, T, S, n_split):
    k = kv()
    d = 128
    print(f"[det] bits={bits} G={G} R={R} B={B} H={H} g={g} T={T} S={S} n_split={n_split}",
          flush=True)
    w = W.Workload("det", 98, 1, B, H, H * g, d, T, bits, G, d, R)
    dims = det_dims(w, S)
    K, V = rand_kv(B, H, T, d, seed=T + g)
    cache = gpu_prefill(w, dims, K, V, T)
    q = torch.randn((B, H * g, d), device="cuda").to(torch.float16)
    sm = 1 / math.sqrt(d)
    ws = k.new_workspace(dims, T, n_split)
    out = torch.empty((B, H * g, d), dtype=torch.float32, device="cuda")
    k.kivi_decode_attn(dims, cache, 0, T, q, sm, out, ws, n_split=n_split)
    torch.cuda.synchronize()
    first = bits_of(out)
    oc = O.LayerCache(B, H, d, bits, G, d, R, dims.max_tokens, sink=S)
    oc.prefill(K.cpu().numpy(), V.cpu().numpy())
    assert_close(out.cpu().numpy(), oc.attend(q.cpu().numpy(), sm), "deterministic decode")
    for rep in range(4):
        k.kivi_decode_attn(dims, cache, 0, T, q, sm, out, ws, n_split=n_split)
        torch.cuda.synchronize()
        assert np.array_equal(first, bits_of(out)), f"repeat {rep} differs"


def test_deterministic_fused_step_equals_two_calls():
    # kivi_append_decode against kivi_append_flush + kivi_decode_attn: the same bits, at
    # every step across flushes
    k = kv()
    d, B, H, g, R = 128, 2, 2, 4, 64
    Tp, steps = 4 * R - 5, R + 9
    w = W.Workload("detf", 99, 1, B, H, H * g, d, Tp + steps, 2, 32, d, R)
    dims = det_dims(w)
    K, V = rand_kv(B, H, Tp + steps, d, seed=5)
    a = gpu_prefill(w, dims, K, V, Tp)
    b_ = gpu_prefill(w, dims, K, V, Tp)
    wa, wb = k.new_workspace(dims, Tp + steps), k.new_workspace(dims, Tp + steps)
    oa = torch.empty((B, H * g, d), dtype=torch.float32, device="cuda")
    ob = torch.empty_like(oa)
    for t in range(Tp, Tp + steps):
        q = torch.randn((B, H * g, d), device="cuda").to(torch.float16)
        kn, vn = K[:, :, t].contiguous(), V[:, :, t].contiguous()
        k.kivi_append_flush(dims, a, 0, t, kn, vn)
        k.kivi_decode_attn(dims, a, 0, t + 1, q, 0.09, oa, wa)
        k.kivi_append_decode(dims, b_, 0, t, kn, vn, q, 0.09, ob, wb)
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(oa), bits_of(ob)), f"step {t}"


@pytest.mark.parametrize("name", ["llama8b_128k_2bit", "llama70b_stream"])
def test_deterministic_full_size(name):
    # the benchmark's shapes in their default launch: repeated calls, same bits; sampled
    # pairs against the oracle
    k = kv()
    w = W.get(name)
    print(f"[det] workload {name}", flush=True)
    dims = det_dims(w)
    K, V = W.make_kv(w, 0, device="cuda", total_tokens=w.tokens)
    cache = gpu_prefill(w, dims, K, V, w.tokens)
    q = W.make_q(w, 0, 0, device="cuda")
    ws = k.new_workspace(dims, w.tokens)
    out = torch.empty((w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    k.kivi_decode_attn(dims, cache, 0, w.tokens, q, w.sm_scale, out, ws)
    torch.cuda.synchronize()
    first = bits_of(out)
    for _ in range(3):
        k.kivi_decode_attn(dims, cache, 0, w.tokens, q, w.sm_scale, out, ws)
        torch.cuda.synchronize()
        assert np.array_equal(first, bits_of(out))
    g = w.gqa
    qh = q.cpu().numpy()
    o = out.cpu().numpy()
    for b, h in [(0, 0), (w.batch - 1, w.kv_heads - 1)]:
        oc = O.LayerCache(1, 1, w.head_dim, w.bits, w.group_k, w.group_v, w.residual,
                          dims.max_tokens)
        oc.prefill(K[b:b + 1, h:h + 1].cpu().numpy(), V[b:b + 1, h:h + 1].cpu().numpy())
        ref = oc.attend(qh[b:b + 1, h * g:(h + 1) * g], w.sm_scale)
        assert_close(o[b, h * g:(h + 1) * g], ref[0], f"{name} pair {(b, h)}")
