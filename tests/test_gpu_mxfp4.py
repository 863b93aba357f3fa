"""GPU parity of the MXFP4 KV codec: the HIP kernels through the C ABI against the CPU
oracle (oracle/mxfp4_ref.py).

Bar: element codes and E8M0 scale codes bit-exact (Key rows, Value runs, including the
zero codes and scales past T in the last run); attention within
|gpu - ref| <= 2e-3 + 1e-3 |ref| elementwise against the oracle's float64 attention
over the same codes.
"""
import numpy as np
import pytest

import oracle as O
import workloads as W
from tests.test_gpu_parity import assert_close

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

D = 128


def kv():
    from bit_quantization_amd import kivi
    return kivi


def mx_inputs(B, H, T, seed, scale=3.0):
    """float16 K/V with an outlier channel and token, a block of zeros, blocks of tiny
    values (scales far below 1), values at the float16 limit, ties and -0."""
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((B, H, T, D)) * scale
    V = rng.standard_normal((B, H, T, D)) * scale
    K[:, :, :, 3] *= 60
    V[:, :, T // 3] *= 200
    K[:, :, :, 32:64] *= 1e-5                  # a block of small values
    V[:, :, :, 96:128] = 0.0                   # a block of zeros
    if T > 2:
        K[:, :, 1, :32] = 65504.0
        V[:, :, 2, 5] = -0.0
        K[:, :, 2, 64:96] = np.array([6, 5, 3.5, 2.5, 1.75, 1.25, 0.75, 0.25] * 4)  # ties
    return K.astype(np.float16), V.astype(np.float16)


def build(B, H, g, T, seed, Tmax=None):
    k = kv()
    Tmax = Tmax or ((T + 40) // 32 + 1) * 32
    dims = k.MxDims(1, B, H, H * g, D, Tmax)
    cache = k.MxCache(dims)
    K, V = mx_inputs(B, H, T, seed)
    k.kivi_mxfp4_quantize(dims, cache, 0, torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda(), T)
    oc = O.MXFP4Cache(B, H, D, Tmax)
    oc.prefill(K, V)
    return dims, cache, oc, K, V


def compare_codes(cache, oc, T):
    nr = (T + 31) // 32
    assert np.array_equal(cache.view("k")[0, :, :, :T].cpu().numpy(), O.pack_nibbles(oc.k[:, :, :T])), \
        "Key codes differ"
    assert np.array_equal(cache.view("k_scale")[0, :, :, :T].cpu().numpy(), oc.ks[:, :, :T]), \
        "Key scales differ"
    assert np.array_equal(cache.view("v")[0, :, :, :nr].cpu().numpy(),
                          O.pack_mx_value_runs(oc.v[:, :, :nr * 32])), "Value runs differ"
    assert np.array_equal(cache.view("v_scale")[0, :, :, :nr].cpu().numpy(),
                          O.pack_value_scales(oc.vs[:, :, :nr * 32])), "Value scales differ"


@pytest.mark.parametrize("B,H,T", [(1, 1, 64), (2, 3, 77), (1, 2, 1), (2, 2, 1000), (1, 1, 33)])
def test_mxfp4_codes_bit_exact(B, H, T):
    dims, cache, oc, _, _ = build(B, H, 2, T, seed=T)
    torch.cuda.synchronize()
    compare_codes(cache, oc, T)


def test_mxfp4_append_equals_prefill():
    k = kv()
    B, H, g, T0, T = 2, 2, 4, 30, 100
    dims, cache, oc, K, V = build(B, H, g, T, seed=5)
    c2 = k.MxCache(dims)
    Kt, Vt = torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda()
    k.kivi_mxfp4_quantize(dims, c2, 0, Kt[:, :, :T0].contiguous(), Vt[:, :, :T0].contiguous(), T0)
    for t in range(T0, T):
        k.kivi_mxfp4_append(dims, c2, 0, t, Kt[:, :, t].contiguous(), Vt[:, :, t].contiguous())
    torch.cuda.synchronize()
    compare_codes(c2, oc, T)


DECODE = [
    # B, H, g, T, n_split
    (1, 1, 1, 1, 0), (2, 3, 4, 1000, 0), (2, 3, 4, 1000, 3), (1, 2, 8, 777, 0), (1, 1, 2, 33, 1),
    (2, 2, 2, 1281, 0), (1, 1, 8, 4096, 0), (3, 1, 1, 96, 2), (1, 8, 4, 20000, 0),
    (1, 2, 4, 4096, 40), (1, 1, 8, 4096, 37),   # merges in several rounds
]


@pytest.mark.parametrize("B,H,g,T,n_split", DECODE)
def test_mxfp4_decode_matches_oracle(B, H, g, T, n_split):
    k = kv()
    dims, cache, oc, _, _ = build(B, H, g, T, seed=T + g)
    gq = torch.Generator(device="cuda")
    gq.manual_seed(T)
    q = torch.randn((B, H * g, D), generator=gq, device="cuda").to(torch.float16)
    out = torch.empty((B, H * g, D), dtype=torch.float32, device="cuda")
    ws = k.new_mxfp4_workspace(dims, T, n_split)
    sm = 1 / np.sqrt(D)
    k.kivi_mxfp4_decode_attn(dims, cache, 0, T, q, sm, out, ws, n_split)
    torch.cuda.synchronize()
    ref = oc.attend(q.cpu().numpy(), sm)
    assert_close(out.cpu().numpy(), ref, f"mxfp4 decode B={B} H={H} g={g} T={T} split={n_split}")
    assert int(torch.count_nonzero(ws[:B * H * 256])) == 0, "arrival counters not reset"


def test_mxfp4_step_matches_oracle_as_tokens_arrive():
    # append + decode steps from a short prompt across several 32-token runs
    k = kv()
    B, H, g = 2, 2, 4
    T0, steps = 5, 70
    dims, cache, oc, K, V = build(B, H, g, T0 + steps, seed=9)
    c2 = k.MxCache(dims)
    Kt, Vt = torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda()
    k.kivi_mxfp4_quantize(dims, c2, 0, Kt[:, :, :T0].contiguous(), Vt[:, :, :T0].contiguous(), T0)
    o2 = O.MXFP4Cache(B, H, D, dims.max_tokens)
    o2.prefill(K[:, :, :T0], V[:, :, :T0])
    ws = k.new_mxfp4_workspace(dims, T0 + steps)
    out = torch.empty((B, H * g, D), dtype=torch.float32, device="cuda")
    gq = torch.Generator(device="cuda")
    gq.manual_seed(1)
    for t in range(T0, T0 + steps):
        q = torch.randn((B, H * g, D), generator=gq, device="cuda").to(torch.float16)
        k.prepare_mxfp4_step(dims, c2, 0, t, Kt[:, :, t].contiguous(), Vt[:, :, t].contiguous(), q,
                             0.09, out, ws)()
        o2.append(K[:, :, t], V[:, :, t])
        if t % 17 == 0 or t == T0 + steps - 1:
            torch.cuda.synchronize()
            assert_close(out.cpu().numpy(), o2.attend(q.cpu().numpy(), 0.09), f"step {t}")


def test_mxfp4_workload_32k_sampled_pairs():
    # the 8B-shaped 32k workload stored as MXFP4, decoded at full size in the default
    # launch; sampled (sequence, KV head) pairs recomputed by the oracle
    k = kv()
    w = W.get("llama8b_32k")
    print("[parity] mxfp4 workload llama8b_32k", flush=True)
    Kd, Vd = W.make_kv(w, 0, device="cuda", total_tokens=w.tokens)
    dims = k.MxDims(1, w.batch, w.kv_heads, w.q_heads, D, w.tokens)
    cache = k.MxCache(dims)
    k.kivi_mxfp4_quantize(dims, cache, 0, Kd, Vd, w.tokens)
    q = W.make_q(w, 0, 0, device="cuda")
    out = torch.empty((w.batch, w.q_heads, D), dtype=torch.float32, device="cuda")
    ws = k.new_mxfp4_workspace(dims, w.tokens)
    k.kivi_mxfp4_decode_attn(dims, cache, 0, w.tokens, q, w.sm_scale, out, ws)
    torch.cuda.synchronize()
    g = w.gqa
    for b, h in [(0, 0), (3, 5), (7, 7)]:
        oc = O.MXFP4Cache(1, 1, D, w.tokens)
        oc.prefill(Kd[b:b + 1, h:h + 1].cpu().numpy(), Vd[b:b + 1, h:h + 1].cpu().numpy())
        assert np.array_equal(cache.view("k")[0, b, h].cpu().numpy(), O.pack_nibbles(oc.k[0, 0]))
        assert np.array_equal(cache.view("v_scale")[0, b, h].cpu().numpy(),
                              O.pack_value_scales(oc.vs[0, 0]))
        ref = oc.attend(q[b:b + 1, h * g:(h + 1) * g].cpu().numpy(), w.sm_scale)
        assert_close(out[b, h * g:(h + 1) * g].cpu().numpy(), ref[0], f"mxfp4 32k pair {(b, h)}")


def test_mxfp4_append_decode_equals_append_then_decode():
    # the one-launch step against kivi_mxfp4_append + kivi_mxfp4_decode_attn on a second
    # cache: outputs to float32 rounding, caches bit-identical; across run boundaries and
    # with several workgroups per pair
    k = kv()
    B, H, g = 2, 2, 4
    T0, steps = 61, 40
    dims, _, _, K, V = build(B, H, g, T0 + steps, seed=13)
    Kt, Vt = torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda()
    a, b_ = k.MxCache(dims), k.MxCache(dims)
    for c in (a, b_):
        k.kivi_mxfp4_quantize(dims, c, 0, Kt[:, :, :T0].contiguous(), Vt[:, :, :T0].contiguous(), T0)
    wa, wb = k.new_mxfp4_workspace(dims, T0 + steps), k.new_mxfp4_workspace(dims, T0 + steps)
    oa = torch.empty((B, H * g, D), dtype=torch.float32, device="cuda")
    ob = torch.empty_like(oa)
    gq = torch.Generator(device="cuda")
    gq.manual_seed(2)
    for t in range(T0, T0 + steps):
        q = torch.randn((B, H * g, D), generator=gq, device="cuda").to(torch.float16)
        kn, vn = Kt[:, :, t].contiguous(), Vt[:, :, t].contiguous()
        k.kivi_mxfp4_append_decode(dims, a, 0, t, kn, vn, q, 0.1, oa, wa)
        k.kivi_mxfp4_append(dims, b_, 0, t, kn, vn)
        k.kivi_mxfp4_decode_attn(dims, b_, 0, t + 1, q, 0.1, ob, wb)
        torch.cuda.synchronize()
        assert np.allclose(oa.cpu().numpy(), ob.cpu().numpy(), rtol=1e-5, atol=1e-6), t
    for name in k.MX_BUFFERS:
        assert torch.equal(a.view(name).cpu(), b_.view(name).cpu()), name
