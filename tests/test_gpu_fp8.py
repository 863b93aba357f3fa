"""GPU parity of the FP8 KV codec: the HIP kernels through the C ABI against the CPU
oracle (oracle/fp8_ref.py).

Bar: FP8 codes bit-exact (Key rows and Value runs, including the zero bytes past T
in the last run); attention within |gpu - ref| <= 2e-3 + 1e-3 |ref| elementwise
against the oracle's float64 attention over the same codes.
"""
import math

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


def fp8_inputs(B, H, T, seed, scale=3.0):
    """float16 K/V with outlier channels and tokens, values past the E4M3 range, tiny
    values that code as subnormals, and -0."""
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((B, H, T, D)) * scale
    V = rng.standard_normal((B, H, T, D)) * scale
    K[:, :, :, 3] *= 60                      # outlier channel (saturates at scale 1)
    V[:, :, T // 3] *= 200                   # outlier token
    K[:, :, :, 7] *= 1e-4                    # subnormal codes
    V[:, :, :, 9] = -0.0
    return K.astype(np.float16), V.astype(np.float16)


def build(fmt, B, H, g, T, k_scale, v_scale, seed, Tmax=None):
    k = kv()
    Tmax = Tmax or ((T + 40) // 32 + 1) * 32
    dims = k.Fp8Dims(1, B, H, H * g, D, fmt, Tmax)
    cache = k.Fp8Cache(dims, k_scale, v_scale)
    K, V = fp8_inputs(B, H, T, seed)
    Kt, Vt = torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda()
    k.kivi_fp8_quantize(dims, cache, 0, Kt, Vt, T)
    oc = O.FP8Cache(B, H, D, fmt, Tmax, k_scale, v_scale)
    oc.prefill(K, V)
    return dims, cache, oc, K, V


def compare_codes(cache, oc, T):
    n_runs = (T + 31) // 32
    gk = cache.view("k")[0, :, :, :T].cpu().numpy()
    assert np.array_equal(gk, oc.k[:, :, :T]), "Key codes differ"
    gv = cache.view("v")[0, :, :, :n_runs].cpu().numpy()
    ref = O.pack_value_runs(oc.v[:, :, :n_runs * 32])
    assert np.array_equal(gv, ref), "Value runs differ"


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("B,H,T,scales", [
    (1, 1, 64, (1.0, 1.0)), (2, 3, 77, ((1.0, 0.37, 2.5), (0.5, 4.0, 1.0))), (1, 2, 1, (1.0, 1.0)),
    (2, 2, 1000, ((0.125, 3.0), (7.0, 0.01))),
])
def test_fp8_codes_bit_exact(fmt, B, H, T, scales):
    dims, cache, oc, _, _ = build(fmt, B, H, 2, T, scales[0], scales[1], seed=T)
    torch.cuda.synchronize()
    compare_codes(cache, oc, T)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_append_equals_prefill(fmt):
    k = kv()
    B, H, g, T0, T = 2, 2, 4, 30, 100
    dims, cache, oc, K, V = build(fmt, B, H, g, T, (1.0, 0.5), (2.0, 1.0), seed=5)
    c2 = k.Fp8Cache(dims, (1.0, 0.5), (2.0, 1.0))
    Kt, Vt = torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda()
    k.kivi_fp8_quantize(dims, c2, 0, Kt[:, :, :T0].contiguous(), Vt[:, :, :T0].contiguous(), T0)
    for t in range(T0, T):
        k.kivi_fp8_append(dims, c2, 0, t, Kt[:, :, t].contiguous(), Vt[:, :, t].contiguous())
    torch.cuda.synchronize()
    compare_codes(c2, oc, T)


DECODE = [
    # fmt, B, H, g, T, n_split
    ("e4m3", 1, 1, 1, 1, 0), ("e4m3", 2, 3, 4, 1000, 0), ("e4m3", 2, 3, 4, 1000, 3),
    ("e4m3", 1, 2, 8, 777, 0), ("e4m3", 1, 1, 2, 33, 1), ("e5m2", 2, 2, 2, 1281, 0),
    ("e5m2", 1, 1, 8, 4096, 0), ("e5m2", 3, 1, 1, 96, 2), ("e4m3", 1, 8, 4, 20000, 0),
    ("e4m3", 1, 2, 4, 4096, 40), ("e5m2", 1, 1, 8, 4096, 37),   # merges in several rounds
]


@pytest.mark.parametrize("fmt,B,H,g,T,n_split", DECODE)
def test_fp8_decode_matches_oracle(fmt, B, H, g, T, n_split):
    k = kv()
    ks = tuple(0.25 + 0.5 * i for i in range(H))
    vs = tuple(1.5 - 0.1 * i for i in range(H))
    dims, cache, oc, _, _ = build(fmt, B, H, g, T, ks, vs, seed=T + g)
    gq = torch.Generator(device="cuda")
    gq.manual_seed(T)
    q = torch.randn((B, H * g, D), generator=gq, device="cuda").to(torch.float16)
    out = torch.empty((B, H * g, D), dtype=torch.float32, device="cuda")
    ws = k.new_fp8_workspace(dims, T, n_split)
    k.kivi_fp8_decode_attn(dims, cache, 0, T, q, 1 / math.sqrt(D), out, ws, n_split)
    torch.cuda.synchronize()
    ref = oc.attend(q.cpu().numpy(), 1 / math.sqrt(D))
    assert_close(out.cpu().numpy(), ref, f"fp8 decode {fmt} B={B} H={H} g={g} T={T} split={n_split}")
    assert int(torch.count_nonzero(ws[:B * H * 256])) == 0, "arrival counters not reset"


def test_fp8_workload_32k_sampled_pairs():
    # the 8B-shaped 32k workload stored as E4M3 with per-head scales from the data's
    # largest magnitude (a calibration on the synthetic data), decoded at full size;
    # sampled (sequence, KV head) pairs recomputed by the oracle
    k = kv()
    w = W.get("llama8b_32k")
    print("[parity] fp8 workload llama8b_32k", flush=True)
    Kd, Vd = W.make_kv(w, 0, device="cuda", total_tokens=w.tokens)
    ks = (Kd.float().abs().amax(dim=(0, 2, 3)) / 448).clamp_min(1e-8).cpu().numpy()
    vs = (Vd.float().abs().amax(dim=(0, 2, 3)) / 448).clamp_min(1e-8).cpu().numpy()
    dims = k.Fp8Dims(1, w.batch, w.kv_heads, w.q_heads, D, "e4m3", w.tokens)
    cache = k.Fp8Cache(dims, ks, vs)
    k.kivi_fp8_quantize(dims, cache, 0, Kd, Vd, w.tokens)
    q = W.make_q(w, 0, 0, device="cuda")
    out = torch.empty((w.batch, w.q_heads, D), dtype=torch.float32, device="cuda")
    ws = k.new_fp8_workspace(dims, w.tokens)
    k.kivi_fp8_decode_attn(dims, cache, 0, w.tokens, q, w.sm_scale, out, ws)
    torch.cuda.synchronize()
    g = w.gqa
    for b, h in [(0, 0), (3, 5), (7, 7)]:
        oc = O.FP8Cache(1, 1, D, "e4m3", w.tokens, ks[h:h + 1], vs[h:h + 1])
        oc.prefill(Kd[b:b + 1, h:h + 1].cpu().numpy(), Vd[b:b + 1, h:h + 1].cpu().numpy())
        assert np.array_equal(cache.view("k")[0, b, h].cpu().numpy(), oc.k[0, 0])
        ref = oc.attend(q[b:b + 1, h * g:(h + 1) * g].cpu().numpy(), w.sm_scale)
        assert_close(out[b, h * g:(h + 1) * g].cpu().numpy(), ref[0], f"fp8 32k pair {(b, h)}")
