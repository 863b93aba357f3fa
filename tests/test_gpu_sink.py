"""GPU parity of attention-sink tokens: the first S tokens of every sequence stay in
float16 and the KIVI rules (groups, window, flushes) apply to the tokens after them.

Bar: every cache byte bit-exact against the oracle (oracle/kivi_ref.py, LayerCache with
``sink=S``), attention within |gpu - ref| <= 2e-3 + 1e-3 |ref|.  The float16 buffers
hold the sink rows at [0, S) and the window at [S, S + R).
"""
import math

import numpy as np
import pytest

import oracle as O
import workloads as W
from tests.test_gpu_parity import assert_close, bits16, rand_kv

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

D = 128


def kv():
    from bit_quantization_amd import kivi
    return kivi


def sink_dims(bits, G, Gv, R, S, B, H, g, Tmax, aging="window"):
    return kv().Dims(layers=1, batch=B, kv_heads=H, q_heads=H * g, head_dim=D, bits=bits,
                     group_k=G, group_v=Gv, residual=R, max_tokens=Tmax, sink=S, aging=aging)


def capacity(T, R):
    return (T + R + 127) // 128 * 128 + 128


def prefill(dims, K, V, T):
    k = kv()
    cache = k.Cache(dims)
    k.kivi_quantize_k(dims, cache, 0, K, T, K.shape[2])
    k.kivi_quantize_v(dims, cache, 0, V, T, V.shape[2])
    return cache


def compare_sink_cache(cache, oc, T, seq=None):
    """Every byte the oracle defines at T tokens, for all pairs (or, with ``seq``, for
    sequence ``seq`` of the GPU cache against a one-sequence oracle).  The oracle keeps
    its window oldest first; the GPU keeps window token Tq + i in ring row
    (Tq + i) mod R after the S sink rows."""
    d = cache.dims
    sel = slice(None) if seq is None else slice(seq, seq + 1)

    def view(name):
        return cache.view(name)[0, sel]

    S, R = d.sink, d.residual
    assert oc.T == T and oc.aging == d.aging
    ns = min(T, S)
    Tq = oc.Tq
    r = T - ns - Tq
    where = f"S={S} T={T} aging={d.aging}"
    ring = torch.from_numpy(S + (Tq + np.arange(r, dtype=np.int64)) % R)
    for name, sink_ref, win_ref in (("k_resid", oc.k_sink, oc.k_resid),
                                    ("v_resid", oc.v_sink, oc.v_resid)):
        rows = view(name).cpu()
        assert np.array_equal(bits16(rows[:, :, :ns]), bits16(sink_ref[:, :, :ns])), \
            f"{name} sink rows {where}"
        assert np.array_equal(bits16(rows[:, :, ring]), bits16(win_ref[:, :, :r])), \
            f"{name} window rows {where}"
    g = view("k_codes")[:, :, :Tq].cpu().numpy()
    assert np.array_equal(g, oc.k_codes[:, :, :Tq]), "k_codes " + where
    g = view("v_codes")[:, :, :Tq // 16].cpu().numpy()
    assert np.array_equal(g, oc.v_codes[:, :, :Tq // 16]), "v_codes " + where
    for name, n in (("k_scale", Tq // d.group_k), ("k_zero", Tq // d.group_k),
                    ("v_scale", Tq), ("v_zero", Tq)):
        g = bits16(view(name)[:, :, :n])
        assert np.array_equal(g, bits16(getattr(oc, name)[:, :, :n])), f"{name} {where}"
    sm = view("scale_max").cpu().numpy()
    ks = oc.k_scale[:, :, :Tq // d.group_k].astype(np.float32)
    vs = oc.v_scale[:, :, :Tq].astype(np.float32)
    ref_k = ks.max(axis=(2, 3)) if ks.shape[2] else np.zeros(sm.shape[:2], np.float32)
    ref_v = vs.max(axis=(2, 3)) if vs.shape[2] else np.zeros(sm.shape[:2], np.float32)
    assert np.array_equal(sm[..., 0], ref_k), "scale_max[0] " + where
    assert np.array_equal(sm[..., 1], ref_v), "scale_max[1] " + where


def oracle_cache(bits, G, Gv, R, S, K, V, T, Tmax, aging="window"):
    B, H = K.shape[0], K.shape[1]
    oc = O.LayerCache(B, H, D, bits, G, Gv, R, Tmax, sink=S, aging=aging)
    oc.prefill(K[:, :, :T].cpu().numpy(), V[:, :, :T].cpu().numpy())
    return oc


PREFILL = [
    # bits, G, Gv, R, S, B, H, T
    (2, 32, 128, 32, 4, 2, 2, 3),           # inside the sink
    (2, 32, 128, 32, 4, 1, 2, 4),           # exactly the sink
    (4, 32, 64, 64, 4, 2, 1, 5),            # sink + one window row
    (2, 32, 128, 32, 7, 1, 3, 39),          # sink + a full window, nothing quantized
    (2, 32, 128, 32, 7, 1, 3, 40),          # one window flushed + 1
    (4, 64, 128, 128, 64, 2, 2, 1000),
    (2, 16, 32, 48, 5, 1, 2, 401),
    (4, 16, 16, 16, 1, 1, 1, 97),
]


@pytest.mark.parametrize("bits,G,Gv,R,S,B,H,T", PREFILL)
def test_sink_prefill_is_bit_exact(bits, G, Gv, R, S, B, H, T):
    Tmax = capacity(T, R)
    dims = sink_dims(bits, G, Gv, R, S, B, H, 1, Tmax)
    K, V = rand_kv(B, H, T + 3, D, seed=T + S)
    cache = prefill(dims, K, V, T)
    torch.cuda.synchronize()
    compare_sink_cache(cache, oracle_cache(bits, G, Gv, R, S, K, V, T, Tmax), T)


@pytest.mark.parametrize("bits,G,Gv,R,S", [(2, 32, 128, 32, 4), (4, 32, 64, 64, 7),
                                           (2, 16, 16, 48, 33)])
def test_sink_streaming_appends_equal_prefill(bits, G, Gv, R, S):
    # the stream starts inside the sink, fills it, then crosses several flushes
    B, H = 2, 2
    Tp, T = 2, S + 3 * R + 7
    Tmax = capacity(T, R)
    dims = sink_dims(bits, G, Gv, R, S, B, H, 1, Tmax)
    K, V = rand_kv(B, H, T, D, seed=S + bits)
    k = kv()
    a = prefill(dims, K, V, Tp)
    for t in range(Tp, T):
        k.kivi_append_flush(dims, a, 0, t, K[:, :, t].contiguous(), V[:, :, t].contiguous())
    b_ = prefill(dims, K, V, T)
    torch.cuda.synchronize()
    oc = oracle_cache(bits, G, Gv, R, S, K, V, T, Tmax)
    compare_sink_cache(a, oc, T)
    compare_sink_cache(b_, oc, T)


DECODE = [
    # bits, G, R, S, B, H, g, T
    (2, 32, 32, 4, 1, 1, 1, 3),             # T < S: only sink rows
    (2, 32, 32, 4, 2, 2, 4, 4),             # T = S
    (4, 32, 64, 7, 1, 2, 8, 40),            # sink + window
    (2, 32, 32, 7, 2, 3, 4, 1000),
    (4, 64, 128, 64, 1, 2, 2, 777),
    (2, 64, 64, 4, 2, 1, 8, 1281),
    (2, 32, 128, 1024, 1, 1, 4, 1300),      # the largest sink
]


@pytest.mark.parametrize("bits,G,R,S,B,H,g,T", DECODE)
@pytest.mark.parametrize("n_split", [0, 3])
def test_sink_decode_matches_oracle(bits, G, R, S, B, H, g, T, n_split):
    k = kv()
    Tmax = capacity(T, R)
    dims = sink_dims(bits, G, D, R, S, B, H, g, Tmax)
    K, V = rand_kv(B, H, T, D, seed=T + S, scale=3.0)
    K[:, :, :2] *= 8                        # large early tokens, as sinks are
    cache = prefill(dims, K, V, T)
    gq = torch.Generator(device="cuda")
    gq.manual_seed(T + S)
    q = torch.randn((B, H * g, D), generator=gq, device="cuda").to(torch.float16)
    out = torch.empty((B, H * g, D), dtype=torch.float32, device="cuda")
    ws = k.new_workspace(dims, T, n_split)
    k.kivi_decode_attn(dims, cache, 0, T, q, 1 / math.sqrt(D), out, ws, n_split=n_split)
    torch.cuda.synchronize()
    oc = oracle_cache(bits, G, D, R, S, K, V, T, Tmax)
    ref = oc.attend(q.cpu().numpy(), 1 / math.sqrt(D))
    assert_close(out.cpu().numpy(), ref, f"sink decode S={S} T={T} n_split={n_split}")


# split counts whose merge takes several rounds (32 partials a round, 16 with 8 query
# heads per KV head)
@pytest.mark.parametrize("bits,G,R,S,B,H,g,T,n_split", [
    (2, 32, 128, 1024, 1, 1, 4, 4000, 40),
    (4, 32, 64, 7, 1, 2, 8, 3000, 35),
])
def test_sink_decode_merge_rounds(bits, G, R, S, B, H, g, T, n_split):
    test_sink_decode_matches_oracle(bits, G, R, S, B, H, g, T, n_split)


@pytest.mark.parametrize("bits,G,R,S,g", [(2, 32, 32, 5, 4), (4, 64, 64, 64, 2)])
def test_sink_append_decode_matches_oracle(bits, G, R, S, g):
    # the fused step from inside the sink across the sink boundary and two flushes;
    # the cache ends bit-identical to a prefill of the same tokens
    k = kv()
    B, H = 2, 2
    Tp, steps = 1, S + 2 * R + 5
    T_end = Tp + steps
    Tmax = capacity(T_end, R)
    dims = sink_dims(bits, G, D, R, S, B, H, g, Tmax)
    K, V = rand_kv(B, H, T_end, D, seed=S + g)
    cache = prefill(dims, K, V, Tp)
    ws = k.new_workspace(dims, T_end)
    gq = torch.Generator(device="cuda")
    gq.manual_seed(S)
    out = torch.empty((B, H * g, D), dtype=torch.float32, device="cuda")
    checks = {Tp, S - 1, S, S + R - 1, S + R, T_end - 1}
    for t in range(Tp, T_end):
        q = torch.randn((B, H * g, D), generator=gq, device="cuda").to(torch.float16)
        k.kivi_append_decode(dims, cache, 0, t, K[:, :, t].contiguous(), V[:, :, t].contiguous(),
                             q, 0.09, out, ws)
        if t in checks:
            torch.cuda.synchronize()
            oc = oracle_cache(bits, G, D, R, S, K, V, t + 1, Tmax)
            assert_close(out.cpu().numpy(), oc.attend(q.cpu().numpy(), 0.09), f"fused step {t}")
    torch.cuda.synchronize()
    compare_sink_cache(cache, oracle_cache(bits, G, D, R, S, K, V, T_end, Tmax), T_end)


def test_sink_workload_32k_sampled_pairs():
    # the 8B-shaped 32k workload with 4 sink tokens, decoded at full size in the default
    # launch; sampled (sequence, KV head) pairs recomputed by the oracle
    k = kv()
    w = W.get("llama8b_32k")
    S = 4
    print("[parity] sink workload llama8b_32k S=4", flush=True)
    Tmax = w.max_tokens()
    dims = k.Dims(1, w.batch, w.kv_heads, w.q_heads, w.head_dim, w.bits, w.group_k, w.group_v,
                  w.residual, Tmax, sink=S)
    Kd, Vd = W.make_kv(w, 0, device="cuda", total_tokens=w.tokens)
    cache = prefill(dims, Kd, Vd, w.tokens)
    q = W.make_q(w, 0, 0, device="cuda")
    out = torch.empty((w.batch, w.q_heads, D), dtype=torch.float32, device="cuda")
    ws = k.new_workspace(dims, w.tokens)
    k.kivi_decode_attn(dims, cache, 0, w.tokens, q, w.sm_scale, out, ws)
    torch.cuda.synchronize()
    g = w.gqa
    for b, h in [(0, 0), (5, 3)]:
        oc = O.LayerCache(1, 1, D, w.bits, w.group_k, w.group_v, w.residual, Tmax, sink=S)
        oc.prefill(Kd[b:b + 1, h:h + 1].cpu().numpy(), Vd[b:b + 1, h:h + 1].cpu().numpy())
        Tq = O.quantized_len(w.tokens - S, w.residual)
        assert np.array_equal(cache.view("k_codes")[0, b, h, :Tq].cpu().numpy(), oc.k_codes[0, 0, :Tq])
        assert np.array_equal(bits16(cache.view("k_resid")[0, b, h, :S]), bits16(oc.k_sink[0, 0]))
        ref = oc.attend(q[b:b + 1, h * g:(h + 1) * g].cpu().numpy(), w.sm_scale)
        assert_close(out[b, h * g:(h + 1) * g].cpu().numpy(), ref[0], f"sink 32k pair {(b, h)}")
