"""GPU parity of group-wise aging of the float16 window: a token arriving at a full
window sends only the oldest Key group (G tokens) into the history, so the window
keeps between R - G + 1 and R of the most recent tokens.

Bar: every cache byte bit-exact against the oracle (LayerCache with
``aging="group"``; the GPU window is a ring over its R rows), attention within
|gpu - ref| <= 2e-3 + 1e-3 |ref|.
"""
import math

import numpy as np
import pytest

import oracle as O
import workloads as W
from tests.test_gpu_parity import assert_close, bits16, rand_kv
from tests.test_gpu_sink import capacity, compare_sink_cache, oracle_cache, prefill, sink_dims

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

D = 128


def kv():
    from bit_quantization_amd import kivi
    return kivi


PREFILL = [
    # bits, G, Gv, R, S, B, H, T
    (2, 32, 128, 128, 0, 2, 2, 100),        # window not full yet
    (2, 32, 128, 128, 0, 1, 2, 129),        # one group aged out, ring start 32
    (4, 16, 64, 64, 0, 2, 1, 200),          # ring wraps
    (2, 32, 128, 128, 4, 1, 3, 1000),
    (4, 64, 128, 128, 7, 2, 2, 777),
    (2, 16, 32, 48, 0, 1, 2, 401),
    (2, 32, 128, 32, 0, 1, 1, 97),          # G = R: the window rule
]


@pytest.mark.parametrize("bits,G,Gv,R,S,B,H,T", PREFILL)
def test_aging_prefill_is_bit_exact(bits, G, Gv, R, S, B, H, T):
    Tmax = capacity(T, R)
    dims = sink_dims(bits, G, Gv, R, S, B, H, 1, Tmax, aging="group")
    K, V = rand_kv(B, H, T + 3, D, seed=T + G)
    cache = prefill(dims, K, V, T)
    torch.cuda.synchronize()
    compare_sink_cache(cache, oracle_cache(bits, G, Gv, R, S, K, V, T, Tmax, "group"), T)


@pytest.mark.parametrize("bits,G,Gv,R,S", [(2, 32, 128, 128, 0), (4, 16, 64, 64, 5),
                                           (2, 16, 16, 48, 0), (4, 64, 128, 128, 33)])
def test_aging_streaming_appends_equal_prefill(bits, G, Gv, R, S):
    # appends from a short prompt across many group flushes and ring wraps; checked
    # against the oracle at several points and against a GPU prefill at the end
    k = kv()
    B, H = 2, 2
    Tp, T = 3, S + 3 * R + 2 * G + 5
    Tmax = capacity(T, R)
    dims = sink_dims(bits, G, Gv, R, S, B, H, 1, Tmax, aging="group")
    K, V = rand_kv(B, H, T, D, seed=S + G + bits)
    a = prefill(dims, K, V, Tp)
    checks = {S + R, S + R + 1, S + R + G + 1, T}
    for t in range(Tp, T):
        k.kivi_append_flush(dims, a, 0, t, K[:, :, t].contiguous(), V[:, :, t].contiguous())
        if t + 1 in checks:
            torch.cuda.synchronize()
            compare_sink_cache(a, oracle_cache(bits, G, Gv, R, S, K, V, t + 1, Tmax, "group"),
                               t + 1)
    b_ = prefill(dims, K, V, T)
    torch.cuda.synchronize()
    compare_sink_cache(b_, oracle_cache(bits, G, Gv, R, S, K, V, T, Tmax, "group"), T)


DECODE = [
    # bits, G, R, S, B, H, g, T
    (2, 32, 128, 0, 1, 1, 1, 100),
    (2, 32, 128, 0, 2, 2, 4, 129),          # ring start 32, wraps by one row
    (2, 32, 128, 0, 2, 3, 4, 1000),         # ring start 0
    (4, 32, 64, 4, 1, 2, 8, 777),
    (2, 64, 128, 0, 2, 1, 8, 1281),
    (4, 32, 96, 7, 1, 2, 2, 2000),
]


@pytest.mark.parametrize("bits,G,R,S,B,H,g,T", DECODE)
@pytest.mark.parametrize("n_split", [0, 3])
def test_aging_decode_matches_oracle(bits, G, R, S, B, H, g, T, n_split):
    k = kv()
    Tmax = capacity(T, R)
    dims = sink_dims(bits, G, D, R, S, B, H, g, Tmax, aging="group")
    K, V = rand_kv(B, H, T, D, seed=T + G, scale=3.0)
    K[:, :, :, 9] *= 20
    cache = prefill(dims, K, V, T)
    gq = torch.Generator(device="cuda")
    gq.manual_seed(T + R)
    q = torch.randn((B, H * g, D), generator=gq, device="cuda").to(torch.float16)
    out = torch.empty((B, H * g, D), dtype=torch.float32, device="cuda")
    ws = k.new_workspace(dims, T, n_split)
    k.kivi_decode_attn(dims, cache, 0, T, q, 1 / math.sqrt(D), out, ws, n_split=n_split)
    torch.cuda.synchronize()
    oc = oracle_cache(bits, G, D, R, S, K, V, T, Tmax, "group")
    assert_close(out.cpu().numpy(), oc.attend(q.cpu().numpy(), 1 / math.sqrt(D)),
                 f"aging decode T={T} n_split={n_split}")


# split counts whose merge takes several rounds (32 partials a round, 16 with 8 query
# heads per KV head)
@pytest.mark.parametrize("bits,G,R,S,B,H,g,T,n_split", [
    (2, 32, 128, 0, 1, 2, 4, 4000, 40),
    (4, 32, 96, 7, 1, 1, 8, 3000, 36),
])
def test_aging_decode_merge_rounds(bits, G, R, S, B, H, g, T, n_split):
    test_aging_decode_matches_oracle(bits, G, R, S, B, H, g, T, n_split)


@pytest.mark.parametrize("bits,G,R,S,g", [(2, 32, 128, 0, 4), (4, 32, 64, 6, 2)])
def test_aging_append_decode_matches_oracle(bits, G, R, S, g):
    # the fused step across group flushes and ring wraps, against the oracle at
    # sampled steps; the cache ends bit-identical to the oracle's
    k = kv()
    B, H = 2, 2
    Tp = S + R - 3
    T_end = Tp + R + 2 * G + 4
    Tmax = capacity(T_end, R)
    dims = sink_dims(bits, G, D, R, S, B, H, g, Tmax, aging="group")
    K, V = rand_kv(B, H, T_end, D, seed=R + g)
    cache = prefill(dims, K, V, Tp)
    ws = k.new_workspace(dims, T_end)
    gq = torch.Generator(device="cuda")
    gq.manual_seed(G)
    out = torch.empty((B, H * g, D), dtype=torch.float32, device="cuda")
    checks = {Tp, S + R - 1, S + R, S + R + 1, S + R + G, S + R + G + 1, T_end - 1}
    for t in range(Tp, T_end):
        q = torch.randn((B, H * g, D), generator=gq, device="cuda").to(torch.float16)
        k.kivi_append_decode(dims, cache, 0, t, K[:, :, t].contiguous(), V[:, :, t].contiguous(),
                             q, 0.09, out, ws)
        if t in checks:
            torch.cuda.synchronize()
            oc = oracle_cache(bits, G, D, R, S, K, V, t + 1, Tmax, "group")
            assert_close(out.cpu().numpy(), oc.attend(q.cpu().numpy(), 0.09), f"fused step {t}")
    torch.cuda.synchronize()
    compare_sink_cache(cache, oracle_cache(bits, G, D, R, S, K, V, T_end, Tmax, "group"), T_end)


def test_aging_workload_32k_sampled_pairs():
    # the 8B-shaped 32k workload with group-wise aging, decoded at full size in the
    # default launch; sampled (sequence, KV head) pairs recomputed by the oracle
    k = kv()
    w = W.get("llama8b_32k")
    print("[parity] aging workload llama8b_32k", flush=True)
    Tmax = w.max_tokens()
    T = w.tokens + 40                       # the window mid-ring
    dims = k.Dims(1, w.batch, w.kv_heads, w.q_heads, w.head_dim, w.bits, w.group_k, w.group_v,
                  w.residual, Tmax, aging="group")
    Kd, Vd = W.make_kv(w, 0, device="cuda", total_tokens=T)
    cache = prefill(dims, Kd, Vd, T)
    q = W.make_q(w, 0, 0, device="cuda")
    out = torch.empty((w.batch, w.q_heads, D), dtype=torch.float32, device="cuda")
    ws = k.new_workspace(dims, T)
    k.kivi_decode_attn(dims, cache, 0, T, q, w.sm_scale, out, ws)
    torch.cuda.synchronize()
    g = w.gqa
    for b, h in [(0, 0), (6, 2)]:
        oc = O.LayerCache(1, 1, D, w.bits, w.group_k, w.group_v, w.residual, Tmax, aging="group")
        oc.prefill(Kd[b:b + 1, h:h + 1].cpu().numpy(), Vd[b:b + 1, h:h + 1].cpu().numpy())
        Tq = oc.Tq
        assert Tq % w.residual != 0          # the ring does not start at row 0
        assert np.array_equal(cache.view("k_codes")[0, b, h, :Tq].cpu().numpy(), oc.k_codes[0, 0, :Tq])
        r = T - Tq
        rows = (Tq + np.arange(r)) % w.residual
        assert np.array_equal(bits16(cache.view("v_resid")[0, b, h].cpu()[torch.from_numpy(rows)]),
                              bits16(oc.v_resid[0, 0, :r]))
        ref = oc.attend(q[b:b + 1, h * g:(h + 1) * g].cpu().numpy(), w.sm_scale)
        assert_close(out[b, h * g:(h + 1) * g].cpu().numpy(), ref[0], f"aging 32k pair {(b, h)}")
