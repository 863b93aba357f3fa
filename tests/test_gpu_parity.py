"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: packed codes, scales, zeros and residual rows bit-exact; attention outputs
within |gpu - ref| <= 2e-3 + 1e-3 * |ref| elementwise (the tolerance stated for this
path), where the oracle attends in float64 over the same codes.

Small cases compare every element; the five workload shapes run at full size on
the GPU and compare sampled (sequence, KV head) pairs that the oracle recomputes
from the same float16 inputs.
"""
import math

import numpy as np
import pytest

import oracle as O
import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-3, 1e-3


def kv():
    from bit_quantization_amd import kivi
    return kivi


def dims_of(w: W.Workload, max_tokens=None):
    return kv().Dims(layers=w.layers, batch=w.batch, kv_heads=w.kv_heads, q_heads=w.q_heads,
                     head_dim=w.head_dim, bits=w.bits, group_k=w.group_k, group_v=w.group_v,
                     residual=w.residual, max_tokens=max_tokens or w.max_tokens())


def bits16(a):
    if isinstance(a, torch.Tensor):
        return a.cpu().view(torch.int16).numpy().view(np.uint16)
    return np.ascontiguousarray(a).view(np.uint16)


def assert_close(got, ref, where=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), f"non-finite output {where}"
    err = np.abs(got - ref)
    lim = ATOL + RTOL * np.abs(ref)
    bad = err > lim
    assert not bad.any(), (f"{where}: {bad.sum()} of {bad.size} outside tolerance; worst "
                           f"err {err.max():.3e} at ref {ref.flat[np.argmax(err - lim)]:.4f}")


def compare_pair(cache, layer, b, h, oc, ob, oh, T):
    """Bit-exact comparison of one (b, h) pair of a GPU cache with an oracle cache."""
    d = cache.dims
    Tq = O.quantized_len(T, d.residual)
    r = T - Tq
    where = f"layer {layer} pair ({b},{h}) T={T}"
    g = cache.view("k_codes")[layer, b, h, :Tq].cpu().numpy()
    assert np.array_equal(g, oc.k_codes[ob, oh, :Tq]), "k_codes " + where
    for name, ref in (("k_scale", oc.k_scale), ("k_zero", oc.k_zero)):
        g = bits16(cache.view(name)[layer, b, h, :Tq // d.group_k])
        assert np.array_equal(g, bits16(ref[ob, oh, :Tq // d.group_k])), name + " " + where
    g = cache.view("v_codes")[layer, b, h, :Tq // 16].cpu().numpy()
    assert np.array_equal(g, oc.v_codes[ob, oh, :Tq // 16]), "v_codes " + where
    for name, ref in (("v_scale", oc.v_scale), ("v_zero", oc.v_zero)):
        g = bits16(cache.view(name)[layer, b, h, :Tq])
        assert np.array_equal(g, bits16(ref[ob, oh, :Tq])), name + " " + where
    for name, ref in (("k_resid", oc.k_resid), ("v_resid", oc.v_resid)):
        g = bits16(cache.view(name)[layer, b, h, :r])
        assert np.array_equal(g, bits16(ref[ob, oh, :r])), name + " " + where
    # scale_max: the largest Key and Value scale of the quantized history (0 if none)
    sm = cache.view("scale_max")[layer, b, h].cpu().numpy()
    ks = oc.k_scale[ob, oh, :Tq // d.group_k].astype(np.float32)
    vs = oc.v_scale[ob, oh, :Tq].astype(np.float32)
    assert sm[0] == (ks.max() if ks.size else 0.0), "scale_max[0] " + where
    assert sm[1] == (vs.max() if vs.size else 0.0), "scale_max[1] " + where


def oracle_pair(w, K, V, b, h, T, max_tokens):
    """Oracle cache of a single (b, h) pair prefetched from host float16 K/V."""
    oc = O.LayerCache(1, 1, w.head_dim, w.bits, w.group_k, w.group_v, w.residual, max_tokens)
    oc.prefill(K[b:b + 1, h:h + 1, :T], V[b:b + 1, h:h + 1, :T])
    return oc


def gpu_prefill(w, dims, K, V, T, layer=0):
    k = kv()
    cache = k.Cache(dims)
    ld = K.shape[2]
    k.kivi_quantize_k(dims, cache, layer, K, T, ld)
    k.kivi_quantize_v(dims, cache, layer, V, T, ld)
    return cache


def gpu_decode(dims, cache, layer, T, q, sm, n_split=0):
    k = kv()
    out = torch.empty((dims.batch, dims.q_heads, dims.head_dim), dtype=torch.float32,
                      device="cuda")
    ws = k.new_workspace(dims, T, n_split)
    k.kivi_decode_attn(dims, cache, layer, T, q, sm, out, ws, n_split=n_split)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ws


def rand_kv(B, H, T, d, seed, scale=2.0, device="cuda"):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    K = (torch.randn((B, H, T, d), generator=g, device=device) * scale).to(torch.float16)
    V = (torch.randn((B, H, T, d), generator=g, device=device) * scale).to(torch.float16)
    return K, V


# ----------------------------------------------------------------------------------
# Small shapes: every element
# ----------------------------------------------------------------------------------

SMALL = [
    # bits, G, Gv, R, B, H, g, T
    (2, 32, 128, 32, 1, 1, 1, 256),
    (2, 32, 128, 64, 2, 3, 4, 1000),
    (4, 32, 128, 128, 1, 2, 8, 777),
    (4, 64, 64, 64, 2, 1, 2, 640),
    (2, 16, 32, 48, 1, 2, 1, 401),
    (4, 16, 16, 16, 1, 1, 1, 97),
    (2, 64, 128, 128, 3, 2, 4, 5),      # only residual
    (2, 32, 128, 32, 1, 1, 2, 32),      # exactly one full window, nothing quantized
    (2, 32, 128, 32, 1, 1, 2, 33),      # one quantized window + 1
]


@pytest.mark.parametrize("bits,G,Gv,R,B,H,g,T", SMALL)
def test_prefill_quantization_is_bit_exact(bits, G, Gv, R, B, H, g, T):
    w = W.Workload("small", 90, 2, B, H, H * g, 128, T, bits, G, Gv, R)
    Tmax = w.max_tokens()
    dims = dims_of(w, Tmax)
    K, V = rand_kv(B, H, T, 128, seed=T * 7 + bits)
    Kh, Vh = K.cpu().numpy(), V.cpu().numpy()
    cache = gpu_prefill(w, dims, K, V, T, layer=1)
    torch.cuda.synchronize()
    oc = O.LayerCache(B, H, 128, bits, G, Gv, R, Tmax)
    oc.prefill(Kh, Vh)
    for b in range(B):
        for h in range(H):
            compare_pair(cache, 1, b, h, oc, b, h, T)
    # layer 0 untouched
    assert int(cache.view("k_codes")[0].abs().sum()) == 0


def special_values(n, seed):
    rng = np.random.default_rng(seed)
    raw = rng.integers(0, 0x7C00, size=n, dtype=np.uint16) | (rng.integers(0, 2, size=n,
                                                                            dtype=np.uint16) << 15)
    x = raw.view(np.float16).copy()
    return x


@pytest.mark.parametrize("bits", [2, 4])
def test_quantizer_edge_values_bit_exact(bits):
    """-0, constant groups, float16 subnormals, +-65504 and arbitrary finite bit
    patterns: codes, scales and zeros bit-exact."""
    B, H, T, d, G, R = 1, 4, 256, 128, 32, 32
    rng = np.random.default_rng(bits)
    K = np.zeros((B, H, T, d), np.float16)
    K[0, 0] = special_values(T * d, 1).reshape(T, d)                       # any finite value
    K[0, 1] = (rng.standard_normal((T, d)) * 1e-6).astype(np.float16)     # subnormal ranges
    K[0, 2] = np.float16(-0.0)
    K[0, 2, :, ::3] = np.float16(3.5)                                      # constant channels
    K[0, 2, 100:140, 7] = np.float16(0.0)
    K[0, 2, 200:205] = np.float16(-0.0)                                    # whole rows of +-0
    K[0, 2, 200:205, 1::2] = np.float16(0.0)
    K[0, 3] = rng.choice(np.array([-65504, 65504, 0, -0.0, 1e-7, 6e-8], np.float16), size=(T, d))
    V = K[:, ::-1].copy()
    w = W.Workload("edge", 91, 1, B, H, H, d, T, bits, G, 128, R)
    dims = dims_of(w, w.max_tokens())
    cache = gpu_prefill(w, dims, torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda(), T)
    torch.cuda.synchronize()
    oc = O.LayerCache(B, H, d, bits, G, 128, R, w.max_tokens())
    oc.prefill(K, V)
    for h in range(H):
        compare_pair(cache, 0, 0, h, oc, 0, h, T)


@pytest.mark.parametrize("bits,G,Gv,R", [(2, 32, 128, 32), (4, 32, 64, 64), (2, 16, 16, 48)])
def test_streaming_appends_equal_prefill(bits, G, Gv, R):
    """Appending token by token (with flushes) writes exactly the prefill bytes,
    on the GPU and in the oracle."""
    B, H, d = 2, 2, 128
    Tp, T = R - 3, 3 * R + 7
    w = W.Workload("stream", 92, 1, B, H, H, d, T, bits, G, Gv, R)
    Tmax = w.max_tokens()
    dims = dims_of(w, Tmax)
    K, V = rand_kv(B, H, T, d, seed=11 + bits)
    k = kv()
    a = gpu_prefill(w, dims, K, V, Tp)
    for t in range(Tp, T):
        k.kivi_append_flush(dims, a, 0, t, K[:, :, t].contiguous(), V[:, :, t].contiguous())
    b_ = gpu_prefill(w, dims, K, V, T)
    torch.cuda.synchronize()
    oc = O.LayerCache(B, H, d, bits, G, Gv, R, Tmax)
    oc.prefill(K.cpu().numpy(), V.cpu().numpy())
    for bb in range(B):
        for h in range(H):
            compare_pair(a, 0, bb, h, oc, bb, h, T)
            compare_pair(b_, 0, bb, h, oc, bb, h, T)


DECODE = [
    # bits, G, R, B, H, g, T
    (2, 32, 32, 1, 1, 1, 256),
    (2, 32, 64, 2, 3, 4, 1000),
    (4, 32, 128, 1, 2, 8, 777),
    (2, 64, 64, 2, 2, 2, 1281),
    (4, 64, 128, 1, 1, 1, 129),
    (2, 32, 128, 2, 2, 8, 100),         # residual only, ragged
    (2, 32, 32, 1, 2, 4, 1),            # a single token
    (4, 32, 32, 1, 1, 2, 33),
]


@pytest.mark.parametrize("bits,G,R,B,H,g,T", DECODE)
@pytest.mark.parametrize("n_split", [0, 1, 3])
def test_decode_matches_oracle(bits, G, R, B, H, g, T, n_split):
    d = 128
    w = W.Workload("dec", 93, 1, B, H, H * g, d, T, bits, G, d, R)
    Tmax = w.max_tokens()
    dims = dims_of(w, Tmax)
    K, V = rand_kv(B, H, T, d, seed=T + bits, scale=3.0)
    K[:, :, :, 5] *= 20        # an outlier channel
    cache = gpu_prefill(w, dims, K, V, T)
    gq = torch.Generator(device="cuda")
    gq.manual_seed(T)
    q = torch.randn((B, H * g, d), generator=gq, device="cuda").to(torch.float16)
    sm = 1 / math.sqrt(d)
    out, ws = gpu_decode(dims, cache, 0, T, q, sm, n_split)
    oc = O.LayerCache(B, H, d, bits, G, d, R, Tmax)
    oc.prefill(K.cpu().numpy(), V.cpu().numpy())
    ref = oc.attend(q.cpu().numpy(), sm)
    assert_close(out, ref, f"decode bits={bits} T={T} n_split={n_split}")


# Explicit split counts around the merge's round sizes: rounds of 8, 16 or 32 partials
# (16 at most with 8 query heads per KV head), so 9 and 17 partials take the larger
# round with clamped, zero-weight slots, and 33 or more partials (17 or more at 8 query
# heads) fold in several rounds with the online rescale between them.  Every count is
# below the cap of one workgroup per 64-token block plus one.
MERGE_ROUNDS = [
    # bits, G, R, B, H, g, T, n_split
    (2, 32, 64, 1, 2, 4, 5000, 9),
    (2, 32, 64, 1, 2, 4, 5000, 17),
    (2, 32, 64, 1, 2, 4, 5000, 33),
    (2, 32, 64, 1, 2, 4, 5000, 64),
    (4, 64, 64, 1, 1, 8, 3000, 17),
    (4, 64, 64, 1, 1, 8, 3000, 40),
    (2, 32, 128, 1, 1, 1, 4000, 50),
    (2, 64, 128, 1, 2, 2, 4100, 37),
]


@pytest.mark.parametrize("bits,G,R,B,H,g,T,n_split", MERGE_ROUNDS)
def test_decode_merge_rounds(bits, G, R, B, H, g, T, n_split):
    d = 128
    print(f"[parity] merge rounds bits={bits} G={G} R={R} B={B} H={H} g={g} T={T} "
          f"n_split={n_split}", flush=True)
    w = W.Workload("rounds", 94, 1, B, H, H * g, d, T, bits, G, d, R)
    Tmax = w.max_tokens()
    dims = dims_of(w, Tmax)
    assert n_split <= (T - R) // 64 + 1
    K, V = rand_kv(B, H, T, d, seed=T + n_split, scale=3.0)
    K[:, :, :, 9] *= 20        # an outlier channel
    # one strong key in the middle: the partials' maxima differ widely, so the weights
    # and the rescale between rounds matter
    K[:, :, T // 2 + 3] *= 6
    cache = gpu_prefill(w, dims, K, V, T)
    gq = torch.Generator(device="cuda")
    gq.manual_seed(T + n_split)
    q = torch.randn((B, H * g, d), generator=gq, device="cuda").to(torch.float16)
    sm = 1 / math.sqrt(d)
    out, ws = gpu_decode(dims, cache, 0, T, q, sm, n_split)
    assert int(torch.count_nonzero(ws[:B * H * 256])) == 0, "arrival counters not reset"
    oc = O.LayerCache(B, H, d, bits, G, d, R, Tmax)
    oc.prefill(K.cpu().numpy(), V.cpu().numpy())
    ref = oc.attend(q.cpu().numpy(), sm)
    assert_close(out, ref, f"merge rounds bits={bits} g={g} T={T} n_split={n_split}")


@pytest.mark.parametrize("bits,G,R,g", [(2, 32, 64, 4), (4, 32, 32, 8), (2, 64, 128, 1)])
def test_default_split_across_flushes_with_one_workspace(bits, G, R, g):
    """The fused step at every T from 2 to 700 with one workspace sized for the last
    T: the default split count changes along the way (it falls right after each
    flush), and every output matches the oracle."""
    k = kv()
    d, B, H = 128, 1, 2
    T_end = 700
    w = W.Workload("steps", 94, 1, B, H, H * g, d, T_end, bits, G, d, R)
    Tmax = w.max_tokens()
    dims = dims_of(w, Tmax)
    K, V = rand_kv(B, H, T_end, d, seed=R + g + bits, scale=3.0)
    cache = gpu_prefill(w, dims, K, V, 1)
    ws = k.new_workspace(dims, T_end)
    Kh, Vh = K.cpu().numpy(), V.cpu().numpy()
    oc = O.LayerCache(B, H, d, bits, G, d, R, Tmax)
    oc.prefill(Kh[:, :, :1], Vh[:, :, :1])
    gq = torch.Generator(device="cuda")
    gq.manual_seed(bits + g)
    out = torch.empty((B, H * g, d), dtype=torch.float32, device="cuda")
    splits = set()
    for t in range(1, T_end):
        q = torch.randn((B, H * g, d), generator=gq, device="cuda").to(torch.float16)
        k.kivi_append_decode(dims, cache, 0, t, K[:, :, t].contiguous(), V[:, :, t].contiguous(),
                             q, 0.09, out, ws)
        oc.append(Kh[:, :, t], Vh[:, :, t])
        splits.add(k.kivi_decode_splits(dims, t + 1))
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), oc.attend(q.cpu().numpy(), 0.09), f"T={t + 1}")
    assert len(splits) > 1, splits


@pytest.mark.parametrize("bits,G,R,B,H,g", [(2, 32, 64, 2, 2, 4), (4, 64, 128, 1, 3, 2),
                                             (2, 32, 32, 2, 1, 8)])
def test_append_decode_equals_append_then_decode(bits, G, R, B, H, g):
    # The fused step (one launch between flushes) against kivi_append_flush followed by
    # kivi_decode_attn on a second cache: outputs agree to float32 rounding, the caches
    # end bit-identical, and sampled steps match the oracle.  The stream starts
    # mid-window and crosses several flushes.
    k = kv()
    d = 128
    Tp, steps = R - 5, 2 * R + 9
    w = W.Workload("fused", 96, 1, B, H, H * g, d, Tp + steps, bits, G, d, R)
    Tmax = w.max_tokens()
    dims = dims_of(w, Tmax)
    K, V = rand_kv(B, H, Tp + steps, d, seed=R + g)
    a = gpu_prefill(w, dims, K, V, Tp)
    b_ = gpu_prefill(w, dims, K, V, Tp)
    wa = k.new_workspace(dims, Tp + steps)
    wb = k.new_workspace(dims, Tp + steps)
    gq = torch.Generator(device="cuda")
    gq.manual_seed(g)
    oa = torch.empty((B, H * g, d), dtype=torch.float32, device="cuda")
    ob = torch.empty_like(oa)
    for t in range(Tp, Tp + steps):
        q = torch.randn((B, H * g, d), generator=gq, device="cuda").to(torch.float16)
        kn, vn = K[:, :, t].contiguous(), V[:, :, t].contiguous()
        k.kivi_append_flush(dims, a, 0, t, kn, vn)
        k.kivi_decode_attn(dims, a, 0, t + 1, q, 0.09, oa, wa)
        k.kivi_append_decode(dims, b_, 0, t, kn, vn, q, 0.09, ob, wb)
        torch.cuda.synchronize()
        assert np.allclose(oa.cpu().numpy(), ob.cpu().numpy(), rtol=1e-5, atol=1e-6), f"step {t}"
        if t in (Tp, Tp + R - 1, Tp + steps - 1):
            oc = O.LayerCache(B, H, d, bits, G, d, R, Tmax)
            oc.prefill(K[:, :, :t + 1].cpu().numpy(), V[:, :, :t + 1].cpu().numpy())
            assert_close(ob.cpu().numpy(), oc.attend(q.cpu().numpy(), 0.09), f"fused step {t}")
    for name in k.BUFFERS:
        assert torch.equal(a.view(name).cpu(), b_.view(name).cpu()), f"{name} differs"


def test_decode_in_a_hip_graph_matches_eager():
    # Replays of a captured decode step, with eager work between them, match the eager
    # call every time (the workspace's counters are reset by each launch itself; no
    # memset is recorded).  Then a captured run of fused append+decode steps leaves the
    # same cache bytes as the same steps run eagerly.
    k = kv()
    d, B, H, g, R = 128, 2, 2, 4, 64
    T0, steps = 3 * R - 2, R + 5
    w = W.Workload("graph", 97, 1, B, H, H * g, d, T0 + steps, 2, 32, d, R)
    dims = dims_of(w, w.max_tokens())
    K, V = rand_kv(B, H, T0 + steps, d, seed=5)
    a = gpu_prefill(w, dims, K, V, T0)
    b_ = gpu_prefill(w, dims, K, V, T0)
    q = torch.randn((B, H * g, d), device="cuda").to(torch.float16)
    ws = k.new_workspace(dims, T0 + steps)
    ref = torch.empty((B, H * g, d), dtype=torch.float32, device="cuda")
    k.kivi_decode_attn(dims, a, 0, T0, q, 0.09, ref, ws)
    torch.cuda.synchronize()
    out = torch.zeros_like(ref)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        k.kivi_decode_attn(dims, a, 0, T0, q, 0.09, out, ws)
    for rep in range(4):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert np.allclose(out.cpu().numpy(), ref.cpu().numpy(), rtol=1e-5, atol=1e-6), f"replay {rep}"
        k.kivi_decode_attn(dims, a, 0, T0, q, 0.09, ref, ws)      # eager work in between
        torch.cuda.synchronize()
    del graph
    oa = torch.empty_like(ref)
    wb = k.new_workspace(dims, T0 + steps)
    for t in range(T0, T0 + steps):
        k.kivi_append_decode(dims, a, 0, t, K[:, :, t].contiguous(), V[:, :, t].contiguous(), q,
                             0.09, oa, ws)
    rows = [(K[:, :, t].contiguous(), V[:, :, t].contiguous()) for t in range(T0, T0 + steps)]
    ob = torch.empty_like(ref)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i, t in enumerate(range(T0, T0 + steps)):
            k.kivi_append_decode(dims, b_, 0, t, rows[i][0], rows[i][1], q, 0.09, ob, wb)
    graph.replay()
    torch.cuda.synchronize()
    assert np.allclose(oa.cpu().numpy(), ob.cpu().numpy(), rtol=1e-5, atol=1e-6)
    for name in k.BUFFERS:
        assert torch.equal(a.view(name).cpu(), b_.view(name).cpu()), f"{name} differs"


def test_decode_repeats_to_float32_rounding():
    # Waves take 64-token blocks from a queue, so the order of float additions can
    # change from call to call; the integer parts of the sums are order-free and the
    # float parts agree to float32 rounding.
    d, B, H, g, T = 128, 2, 2, 4, 5000
    w = W.Workload("det", 94, 1, B, H, H * g, d, T, 2, 32, d, 128)
    dims = dims_of(w, w.max_tokens())
    K, V = rand_kv(B, H, T, d, seed=3)
    cache = gpu_prefill(w, dims, K, V, T)
    q = torch.randn((B, H * g, d), device="cuda").to(torch.float16)
    a, _ = gpu_decode(dims, cache, 0, T, q, 0.09)
    for _ in range(3):
        b, _ = gpu_decode(dims, cache, 0, T, q, 0.09)
        assert np.allclose(a, b, rtol=1e-5, atol=1e-6)


def test_decode_workspace_reused_across_shapes():
    # The contract: zero-fill before the first use with a given batch and kv_heads;
    # later calls with those reuse it for any T, split count, q_heads and bits.  Its
    # leading per-pair arrival counters (256 bytes per (sequence, KV head)) are back
    # to zero after every call.
    k = kv()
    groups = [  # (B, H): [(bits, G, R, g, T, n_split), ...]
        ((2, 3), [(2, 32, 64, 4, 1000, 0), (2, 32, 64, 4, 1000, 5), (4, 32, 32, 8, 777, 3),
                  (2, 64, 64, 2, 1281, 0), (2, 32, 64, 4, 999, 2), (2, 32, 64, 4, 1000, 5)]),
        ((3, 1), [(2, 64, 64, 2, 1281, 0), (4, 32, 32, 2, 300, 7), (2, 64, 64, 2, 1281, 0)]),
    ]
    for (B, H), cases in groups:
        size = 0
        for bits, G, R, g, T, n_split in cases:
            w = W.Workload("ws", 95, 1, B, H, H * g, 128, T, bits, G, 128, R)
            size = max(size, k.kivi_decode_workspace_bytes(dims_of(w, w.max_tokens()), T, n_split))
        ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
        for bits, G, R, g, T, n_split in cases:
            where = (B, H, bits, g, T, n_split)
            print(f"[parity] shared workspace {where}", flush=True)
            w = W.Workload("ws", 95, 1, B, H, H * g, 128, T, bits, G, 128, R)
            dims = dims_of(w, w.max_tokens())
            K, V = rand_kv(B, H, T, 128, seed=T + 7 * bits)
            cache = gpu_prefill(w, dims, K, V, T)
            q = torch.randn((B, H * g, 128), device="cuda").to(torch.float16)
            out = torch.empty((B, H * g, 128), dtype=torch.float32, device="cuda")
            k.kivi_decode_attn(dims, cache, 0, T, q, 0.088, out, ws, n_split=n_split)
            torch.cuda.synchronize()
            assert int(torch.count_nonzero(ws[:B * H * 256])) == 0, f"counters not reset {where}"
            oc = O.LayerCache(B, H, 128, bits, G, 128, R, w.max_tokens())
            oc.prefill(K.cpu().numpy(), V.cpu().numpy())
            assert_close(out.cpu().numpy(), oc.attend(q.cpu().numpy(), 0.088),
                         f"shared workspace {where}")


# ----------------------------------------------------------------------------------
# The workload shapes at full size (sampled pairs)
# ----------------------------------------------------------------------------------

def run_workload_layer(w, layer, pairs, check_decode=True, n_split=0):
    """Quantize and decode layer `layer` of a single-layer-cache workload."""
    dims = dims_of(w)
    K, V = W.make_kv(w, layer, device="cuda", total_tokens=w.tokens)
    L = 0
    cache = gpu_prefill(w, dims, K, V, w.tokens, layer=L)
    T = w.tokens
    q = W.make_q(w, layer, 0, device="cuda")
    out = None
    if check_decode:
        out, _ = gpu_decode(dims, cache, L, T, q, w.sm_scale, n_split)
    qh = q.cpu().numpy()
    g = w.gqa
    for b, h in pairs:
        Kh = K[b:b + 1, h:h + 1].cpu().numpy()
        Vh = V[b:b + 1, h:h + 1].cpu().numpy()
        oc = O.LayerCache(1, 1, w.head_dim, w.bits, w.group_k, w.group_v, w.residual,
                          w.max_tokens())
        oc.prefill(Kh, Vh)
        compare_pair(cache, L, b, h, oc, 0, 0, T)
        if check_decode:
            ref = oc.attend(qh[b:b + 1, h * g:(h + 1) * g], w.sm_scale)
            assert_close(out[b, h * g:(h + 1) * g], ref[0], f"{w.name} layer {layer} pair {(b, h)}")
    return dims, cache, K, V


@pytest.mark.parametrize("name,pairs", [
    ("tiny", [(0, 0)]),
    ("llama8b_32k", [(0, 0), (3, 5), (7, 7)]),
    ("llama8b_128k_4bit", [(0, 0), (0, 3), (0, 7)]),
    ("llama8b_128k_2bit", [(0, 1), (0, 6)]),
])
def test_workload_full_size(name, pairs):
    w = W.get(name)
    print(f"[parity] workload {name} pairs {pairs}", flush=True)
    run_workload_layer(w, 0, pairs)


def test_workload_streaming_70b():
    """Prefill 32768 then 256 append+decode steps; decode checked at the flush steps
    (1 and 129), their neighbours and the last step; the final cache equals a
    prefill of all 33024 tokens, bit for bit."""
    w = W.get("llama70b_stream")
    print("[parity] workload llama70b_stream", flush=True)
    k = kv()
    dims = dims_of(w)
    K, V = W.make_kv(w, 0, device="cuda")                 # 33024 tokens drawn up front
    cache = gpu_prefill(w, dims, K, V, w.tokens)
    pairs = [(0, 0), (9, 4), (15, 7)]
    orc = {p: oracle_pair(w, K[p[0]:p[0] + 1, p[1]:p[1] + 1].cpu().numpy(),
                          V[p[0]:p[0] + 1, p[1]:p[1] + 1].cpu().numpy(), 0, 0, w.tokens,
                          w.max_tokens()) for p in pairs}
    check_steps = {1, 2, 128, 129, 130, 256}
    g = w.gqa
    for step in range(1, w.stream_steps + 1):
        T_before = w.tokens + step - 1
        k.kivi_append_flush(dims, cache, 0, T_before, K[:, :, T_before].contiguous(),
                            V[:, :, T_before].contiguous())
        for (b, h), oc in orc.items():
            oc.append(K[b:b + 1, h:h + 1, T_before].cpu().numpy(),
                      V[b:b + 1, h:h + 1, T_before].cpu().numpy())
        if step in check_steps:
            q = W.make_q(w, 0, step, device="cuda")
            out, _ = gpu_decode(dims, cache, 0, T_before + 1, q, w.sm_scale)
            qh = q.cpu().numpy()
            for (b, h), oc in orc.items():
                ref = oc.attend(qh[b:b + 1, h * g:(h + 1) * g], w.sm_scale)
                assert_close(out[b, h * g:(h + 1) * g], ref[0], f"stream step {step} pair {(b, h)}")
            print(f"[parity] stream step {step} ok", flush=True)
    T = w.tokens + w.stream_steps
    for (b, h), oc in orc.items():
        compare_pair(cache, 0, b, h, oc, 0, 0, T)
    full = gpu_prefill(w, dims, K, V, T)
    torch.cuda.synchronize()
    for name in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero"):
        assert torch.equal(cache.buffers[name], full.buffers[name]), name
    Tq = O.quantized_len(T, w.residual)
    r = T - Tq
    assert torch.equal(cache.view("k_resid")[:, :, :, :r], full.view("k_resid")[:, :, :, :r])
    assert torch.equal(cache.view("v_resid")[:, :, :, :r], full.view("v_resid")[:, :, :, :r])


def test_workload_long_1m_all_layers():
    """32 layers x 1M tokens on one GPU: every layer quantized and decoded; the
    oracle checks two KV heads on three of the layers."""
    w = W.get("long_1m")
    k = kv()
    dims = dims_of(w)
    cache = k.Cache(dims)
    T = w.tokens
    outs = []
    sample = {0: [(0, 0), (0, 5)], 17: [(0, 2)], 31: [(0, 7)]}
    g = w.gqa
    for layer in range(w.layers):
        K, V = W.make_kv(w, layer, device="cuda", total_tokens=T)
        k.kivi_quantize_k(dims, cache, layer, K, T, T)
        k.kivi_quantize_v(dims, cache, layer, V, T, T)
        q = W.make_q(w, layer, 0, device="cuda")
        out, _ = gpu_decode(dims, cache, layer, T, q, w.sm_scale)
        outs.append(out)
        if layer in sample:
            qh = q.cpu().numpy()
            for b, h in sample[layer]:
                oc = O.LayerCache(1, 1, w.head_dim, w.bits, w.group_k, w.group_v, w.residual,
                                  w.max_tokens())
                oc.prefill(K[b:b + 1, h:h + 1].cpu().numpy(), V[b:b + 1, h:h + 1].cpu().numpy())
                compare_pair(cache, layer, b, h, oc, 0, 0, T)
                ref = oc.attend(qh[b:b + 1, h * g:(h + 1) * g], w.sm_scale)
                assert_close(out[b, h * g:(h + 1) * g], ref[0], f"1M layer {layer} pair {(b, h)}")
            print(f"[parity] 1M layer {layer} checked", flush=True)
        del K, V
    assert all(np.isfinite(o).all() for o in outs)
