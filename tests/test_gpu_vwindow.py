"""The per-token Value window (KIVI_FLAG_VALUE_TOKEN_WINDOW) on the GPU against the
oracle's LayerCache(..., v_window="token").

"4.4 KV Cache quantization" §3.2: each new Value enters an R-token float16 window and
pushes the oldest one out, which is quantized on its own; Keys keep their rule (whole
window, or group-wise aging).  Bar: every byte of the cache bit-exact (codes, scales,
zeros, sink and window rows, scale_max) at every step of streams that cross Value
slides and Key flushes; attention within |gpu - ref| <= 2e-3 + 1e-3 |ref| of the
oracle's float64 attention over the same codes, at n_split {default, 1, 3}; the
70B-shaped stream at full size on sampled pairs.
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


def vdims(bits, G, Gv, R, S, B, H, g, Tmax, aging="window"):
    return kv().Dims(layers=1, batch=B, kv_heads=H, q_heads=H * g, head_dim=D, bits=bits,
                     group_k=G, group_v=Gv, residual=R, max_tokens=Tmax, sink=S, aging=aging,
                     v_window="token")


def capacity(T, R, G=32):
    m = math.lcm(16, G, R)
    return (T + R + m) // m * m + m


def prefill(dims, K, V, T):
    k = kv()
    cache = k.Cache(dims)
    k.kivi_quantize_k(dims, cache, 0, K, T, K.shape[2])
    k.kivi_quantize_v(dims, cache, 0, V, T, V.shape[2])
    return cache


def oracle(dims, K, V, T, seq=None):
    sel = slice(None) if seq is None else slice(seq, seq + 1)
    Kh, Vh = K[sel, :, :T], V[sel, :, :T]
    if isinstance(Kh, torch.Tensor):
        Kh, Vh = Kh.cpu().numpy(), Vh.cpu().numpy()
    oc = O.LayerCache(Kh.shape[0], Kh.shape[1], D, dims.bits, dims.group_k, dims.group_v,
                      dims.residual, dims.max_tokens, sink=dims.sink, aging=dims.aging,
                      v_window="token")
    oc.prefill(Kh, Vh)
    return oc


def compare(cache, oc, where, pairs=None):
    """Every byte the oracle defines.  The oracle keeps its windows oldest first; the GPU
    keeps window token i (counted after the sink) in ring row S + (i mod R)."""
    d = cache.dims
    S, R, G = d.sink, d.residual, d.group_k
    T = oc.T
    ns = min(T, S)
    Tq, Tqv = oc.Tq, oc.Tqv
    r, rv = oc.Tk - Tq, oc.Tk - Tqv
    B, H = oc.B, oc.H

    def view(name):
        v = cache.view(name)[0]
        if pairs is not None:
            b, h = pairs
            v = v[b:b + 1, h:h + 1]
        return v.cpu()

    for name, sink_ref, win_ref, t0, n in (("k_resid", oc.k_sink, oc.k_resid, Tq, r),
                                           ("v_resid", oc.v_sink, oc.v_resid, Tqv, rv)):
        rows = view(name)
        assert np.array_equal(bits16(rows[:, :, :ns]), bits16(sink_ref[:, :, :ns])), \
            f"{name} sink rows {where}"
        ring = torch.from_numpy(S + (t0 + np.arange(n, dtype=np.int64)) % R)
        assert np.array_equal(bits16(rows[:, :, ring]), bits16(win_ref[:, :, :n])), \
            f"{name} window rows {where}"
    assert np.array_equal(view("k_codes")[:, :, :Tq].numpy(), oc.k_codes[:, :, :Tq]), \
        "k_codes " + where
    nrun = (Tqv + 15) // 16
    assert np.array_equal(view("v_codes")[:, :, :nrun].numpy(), oc.v_codes[:, :, :nrun]), \
        "v_codes " + where
    for name, n in (("k_scale", Tq // G), ("k_zero", Tq // G), ("v_scale", Tqv), ("v_zero", Tqv)):
        assert np.array_equal(bits16(view(name)[:, :, :n]), bits16(getattr(oc, name)[:, :, :n])), \
            f"{name} {where}"
    sm = view("scale_max").numpy()
    ks = oc.k_scale[:, :, :Tq // G].astype(np.float32)
    vs = oc.v_scale[:, :, :Tqv].astype(np.float32)
    ref_k = ks.max(axis=(2, 3)) if ks.shape[2] else np.zeros((B, H), np.float32)
    ref_v = vs.max(axis=(2, 3)) if vs.shape[2] else np.zeros((B, H), np.float32)
    assert np.array_equal(sm[..., 0], ref_k), "scale_max[0] " + where
    assert np.array_equal(sm[..., 1], ref_v), "scale_max[1] " + where


PREFILL = [
    # bits, G, Gv, R, S, aging, B, H, T
    (2, 32, 128, 64, 0, "window", 2, 2, 40),        # Tk < R: nothing quantized yet
    (2, 32, 128, 64, 0, "window", 1, 2, 64),        # Tk = R
    (2, 32, 128, 64, 0, "window", 1, 2, 65),        # one Value quantized
    (4, 32, 64, 64, 0, "window", 2, 1, 64 + 17),    # a partial 16-token run
    (2, 32, 128, 128, 4, "window", 1, 2, 1000),
    (4, 64, 128, 128, 0, "group", 2, 2, 777),
    (2, 16, 32, 48, 5, "group", 1, 2, 401),
    (4, 16, 16, 16, 1, "window", 1, 1, 97),
]


@pytest.mark.parametrize("bits,G,Gv,R,S,aging,B,H,T", PREFILL)
def test_vwindow_prefill_is_bit_exact(bits, G, Gv, R, S, aging, B, H, T):
    dims = vdims(bits, G, Gv, R, S, B, H, 1, capacity(T, R, G), aging)
    K, V = rand_kv(B, H, T, D, seed=T + R)
    cache = prefill(dims, K, V, T)
    torch.cuda.synchronize()
    compare(cache, oracle(dims, K, V, T), f"prefill T={T} S={S} aging={aging}")


@pytest.mark.parametrize("bits,G,Gv,R,S,aging", [
    (2, 32, 128, 64, 0, "window"), (4, 32, 64, 64, 3, "group"), (2, 16, 16, 32, 0, "window"),
])
def test_vwindow_appends_match_oracle_every_step(bits, G, Gv, R, S, aging):
    # from inside the sink (or an empty window) across Value slides, Key flushes and
    # partial Value runs, every byte checked after every append; the end equals prefill
    k = kv()
    B, H = 2, 2
    T0, T1 = 1, S + 3 * R + 19
    dims = vdims(bits, G, Gv, R, S, B, H, 1, capacity(T1, R, G), aging)
    K, V = rand_kv(B, H, T1, D, seed=7 * R + bits)
    cache = prefill(dims, K, V, T0)
    Kh, Vh = K.cpu().numpy(), V.cpu().numpy()
    oc = O.LayerCache(B, H, D, bits, G, Gv, R, dims.max_tokens, sink=S, aging=aging,
                      v_window="token")
    oc.prefill(Kh[:, :, :T0], Vh[:, :, :T0])
    for t in range(T0, T1):
        k.kivi_append_flush(dims, cache, 0, t, K[:, :, t].contiguous(), V[:, :, t].contiguous())
        torch.cuda.synchronize()
        oc.append(Kh[:, :, t], Vh[:, :, t])
        compare(cache, oc, f"append T={t + 1}")
    compare(prefill(dims, K, V, T1), oc, f"prefill T={T1}")


DECODE = [
    # bits, G, R, S, aging, B, H, g, T
    (2, 32, 128, 0, "window", 2, 2, 4, 1000),
    (2, 32, 128, 0, "window", 1, 2, 4, 128 + 64 * 7 + 3),   # Tqv a multiple of 64 plus 3
    (4, 32, 64, 0, "window", 2, 3, 8, 777),
    (2, 64, 128, 4, "group", 1, 2, 2, 2000),
    (4, 32, 32, 0, "window", 1, 1, 1, 33),                   # one quantized Value
    (2, 32, 64, 0, "window", 2, 2, 4, 64),                   # no quantized Value
    (2, 32, 128, 0, "group", 1, 2, 8, 5003),
]


@pytest.mark.parametrize("bits,G,R,S,aging,B,H,g,T", DECODE)
@pytest.mark.parametrize("n_split", [0, 1, 3])
def test_vwindow_decode_matches_oracle(bits, G, R, S, aging, B, H, g, T, n_split):
    k = kv()
    dims = vdims(bits, G, D, R, S, B, H, g, capacity(T, R, G), aging)
    K, V = rand_kv(B, H, T, D, seed=T + g, scale=3.0)
    K[:, :, :, 5] *= 20
    cache = prefill(dims, K, V, T)
    q = torch.randn((B, H * g, D), device="cuda").to(torch.float16)
    sm = 1 / math.sqrt(D)
    out = torch.empty((B, H * g, D), dtype=torch.float32, device="cuda")
    ws = k.new_workspace(dims, T, n_split)
    k.kivi_decode_attn(dims, cache, 0, T, q, sm, out, ws, n_split=n_split)
    torch.cuda.synchronize()
    oc = oracle(dims, K, V, T)
    assert_close(out.cpu().numpy(), oc.attend(q.cpu().numpy(), sm),
                 f"vwindow decode T={T} n_split={n_split}")


# split counts whose merge takes several rounds (32 partials a round, 16 with 8 query
# heads per KV head)
@pytest.mark.parametrize("bits,G,R,S,aging,B,H,g,T,n_split", [
    (2, 32, 128, 0, "window", 2, 2, 4, 5000, 40),
    (2, 32, 128, 0, "group", 1, 2, 8, 5003, 37),
])
def test_vwindow_decode_merge_rounds(bits, G, R, S, aging, B, H, g, T, n_split):
    test_vwindow_decode_matches_oracle(bits, G, R, S, aging, B, H, g, T, n_split)


@pytest.mark.parametrize("bits,G,R,aging,g,S", [
    (2, 32, 64, "window", 4, 0),
    (4, 64, 128, "group", 8, 0),
    (2, 32, 32, "window", 2, 3),    # R < 64: ring rows recur inside one 64-token span
    (4, 32, 64, "group", 4, 5),
])
def test_vwindow_fused_step_matches_oracle(bits, G, R, aging, g, S):
    # kivi_append_decode from inside the first window across slides and flushes: most
    # steps are one decode launch that quantizes the leaving Value itself; steps that
    # flush Keys, or whose leaving Value completes a 64-token block, launch the append
    # first.  Outputs and every cache byte against the oracle at every step.
    k = kv()
    B, H = 2, 2
    Tp = S + R - 7
    T1 = Tp + 2 * R + 70
    dims = vdims(bits, G, D, R, S, B, H, g, capacity(T1, R, G), aging)
    print(f"[vwindow] fused bits={bits} G={G} R={R} aging={aging} g={g} S={S}", flush=True)
    K, V = rand_kv(B, H, T1, D, seed=R + g + S)
    cache = prefill(dims, K, V, Tp)
    Kh, Vh = K.cpu().numpy(), V.cpu().numpy()
    oc = O.LayerCache(B, H, D, bits, G, D, R, dims.max_tokens, sink=S, aging=aging,
                      v_window="token")
    oc.prefill(Kh[:, :, :Tp], Vh[:, :, :Tp])
    ws = k.new_workspace(dims, T1)
    out = torch.empty((B, H * g, D), dtype=torch.float32, device="cuda")
    for t in range(Tp, T1):
        q = torch.randn((B, H * g, D), device="cuda").to(torch.float16)
        k.kivi_append_decode(dims, cache, 0, t, K[:, :, t].contiguous(), V[:, :, t].contiguous(),
                             q, 0.09, out, ws)
        torch.cuda.synchronize()
        oc.append(Kh[:, :, t], Vh[:, :, t])
        assert_close(out.cpu().numpy(), oc.attend(q.cpu().numpy(), 0.09), f"fused step T={t + 1}")
        compare(cache, oc, f"fused step T={t + 1}")


@pytest.mark.parametrize("bits,G,R,aging,S", [(2, 32, 64, "window", 0), (4, 32, 32, "group", 2)])
def test_vwindow_fused_step_equals_two_launches(bits, G, R, aging, S):
    # with KIVI_FLAG_DETERMINISTIC, kivi_append_decode (one launch on most steps) and
    # kivi_append_flush + kivi_decode_attn give the same output bits and cache bytes at
    # every step: the decode's own quantization of the leaving Value writes what the
    # append kernel writes, and attends with the values the codes give
    k = kv()
    B, H, g = 2, 2, 4
    Tp = S + R - 3
    T1 = Tp + 2 * R + 70
    dims = vdims(bits, G, D, R, S, B, H, g, capacity(T1, R, G), aging)
    dims.deterministic = True
    K, V = rand_kv(B, H, T1, D, seed=11 + R)
    a = prefill(dims, K, V, Tp)
    b_ = prefill(dims, K, V, Tp)
    wa, wb = k.new_workspace(dims, T1), k.new_workspace(dims, T1)
    oa = torch.empty((B, H * g, D), dtype=torch.float32, device="cuda")
    ob = torch.empty_like(oa)
    names = ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero", "k_resid",
             "v_resid", "scale_max")
    for t in range(Tp, T1):
        q = torch.randn((B, H * g, D), device="cuda").to(torch.float16)
        kn, vn = K[:, :, t].contiguous(), V[:, :, t].contiguous()
        k.kivi_append_flush(dims, a, 0, t, kn, vn)
        k.kivi_decode_attn(dims, a, 0, t + 1, q, 0.09, oa, wa)
        k.kivi_append_decode(dims, b_, 0, t, kn, vn, q, 0.09, ob, wb)
        torch.cuda.synchronize()
        assert np.array_equal(oa.cpu().numpy().view(np.uint32), ob.cpu().numpy().view(np.uint32)), \
            f"output bits, step T={t + 1}"
        for n in names:
            assert torch.equal(a.view(n), b_.view(n)), f"{n}, step T={t + 1}"


def test_vwindow_70b_stream_full_size():
    # the 70B-shaped streaming workload (batch 16, GQA 8:1, 32768-token prompt, 256
    # append + decode steps) with the per-token Value window; sampled pairs against the
    # oracle at the first, a flush and the last step, and their bytes at the end
    k = kv()
    w = W.get("llama70b_stream")
    print("[vwindow] llama70b_stream full size", flush=True)
    Tmax = w.max_tokens()
    dims = vdims(w.bits, w.group_k, w.group_v, w.residual, 0, w.batch, w.kv_heads, w.gqa, Tmax)
    K, V = W.make_kv(w, 0, device="cuda", total_tokens=w.total_tokens)
    cache = prefill(dims, K, V, w.tokens)
    ws = k.new_workspace(dims, w.total_tokens)
    out = torch.empty((w.batch, w.q_heads, D), dtype=torch.float32, device="cuda")
    pairs = [(0, 0), (7, 3), (15, 7)]
    g = w.gqa
    checks = {w.tokens, w.tokens + 127, w.total_tokens - 1}
    for t in range(w.tokens, w.total_tokens):
        q = W.make_q(w, 0, t - w.tokens, device="cuda")
        k.kivi_append_decode(dims, cache, 0, t, K[:, :, t].contiguous(), V[:, :, t].contiguous(),
                             q, w.sm_scale, out, ws)
        if t in checks:
            torch.cuda.synchronize()
            o = out.cpu().numpy()
            qh = q.cpu().numpy()
            for b, h in pairs:
                oc = oracle(dims, K[:, h:h + 1], V[:, h:h + 1], t + 1, seq=b)
                ref = oc.attend(qh[b:b + 1, h * g:(h + 1) * g], w.sm_scale)
                assert_close(o[b, h * g:(h + 1) * g], ref[0], f"70B step T={t + 1} pair {(b, h)}")
    torch.cuda.synchronize()
    for b, h in pairs:
        oc = oracle(dims, K[:, h:h + 1], V[:, h:h + 1], w.total_tokens, seq=b)
        compare(cache, oc, f"70B end pair {(b, h)}", pairs=(b, h))
