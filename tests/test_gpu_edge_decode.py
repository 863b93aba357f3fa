"""Decode attention over caches built from the quantizer's edge cases, against the oracle.

The cache bytes of these inputs are checked bit for bit in test_gpu_parity.py; here
the decode reads them: the kernel writes the query side of each product in 32-bit fixed
point with exponents taken from the pair's largest Key and Value scale, so its extremes
are exercised by
  * arbitrary finite float16 bit patterns and +-65504 (scales near the float16 maximum,
    logits in the tens of thousands),
  * a pair whose every Key group and Value group is constant (every scale 0, the
    exponent falls back to 0, the zeros alone carry the values),
  * a pair whose scales are all float16 subnormals, with a query small enough that the
    Key-side exponent reaches its cap of 60,
  * -0, constant channels, whole rows of +-0 and subnormal ranges.
Bar: |gpu - ref| <= 2e-3 + 1e-3 |ref| elementwise, the oracle attending in float64
over the same codes; bits {2, 4}, n_split {default, 1, 3}, then fused append + decode
steps across a flush.
"""
import math

import numpy as np
import pytest

import oracle as O
import workloads as W
from tests.test_gpu_parity import assert_close, dims_of, gpu_prefill, special_values

torch = pytest.importorskip("torch")

B, H, D, G, R = 1, 6, 128, 32, 32
T0 = 256                   # prompt: 224 quantized tokens and a full window of 32
EXTRA = 40                 # rows for the appended tokens


def edge_inputs(bits):
    """K, V float16 [1, 6, T0 + EXTRA, 128] and q float16 [1, 6, 128] (one query head per
    KV head, so each head's query can be scaled on its own)."""
    rng = np.random.default_rng(100 + bits)
    T = T0 + EXTRA
    K = np.zeros((B, H, T, D), np.float16)
    K[0, 0] = special_values(T * D, 1 + bits).reshape(T, D)              # any finite value
    K[0, 1] = (rng.standard_normal((T, D)) * 1e-6).astype(np.float16)   # subnormal ranges
    K[0, 2] = np.float16(-0.0)
    K[0, 2, :, ::3] = np.float16(3.5)                                    # constant channels
    K[0, 2, 100:140, 7] = np.float16(0.0)
    K[0, 2, 200:205] = np.float16(-0.0)                                  # whole rows of +-0
    K[0, 2, 200:205, 1::2] = np.float16(0.0)
    K[0, 3] = rng.choice(np.array([-65504, 65504, 0, -0.0, 1e-7, 6e-8], np.float16), size=(T, D))
    V = K[:, [3, 2, 1, 0, 0, 0]].copy()
    # head 4: every Key group (32 tokens of one channel) and every Value group (one
    # token's 128 channels) constant, so every scale is 0
    kc = (rng.standard_normal((T // G + 1, D)) * 3).astype(np.float16)
    K[0, 4] = np.repeat(kc, G, axis=0)[:T]
    V[0, 4] = (rng.standard_normal((T, 1)) * 3).astype(np.float16)
    # head 5: integer multiples of 2^-24 in [-8, 7]: ranges of at most 15 * 2^-24, so every
    # scale is a float16 subnormal
    tiny = np.float16(2.0 ** -24)
    K[0, 5] = (rng.integers(-8, 8, size=(T, D)) * tiny).astype(np.float16)
    V[0, 5] = (rng.integers(-8, 8, size=(T, D)) * tiny).astype(np.float16)
    q = rng.standard_normal((B, H, D)).astype(np.float32)
    # head 5's query: |q| sm_scale log2(e) times the largest Key scale falls below
    # 2^-30, so the Key-side fixed-point exponent is capped at 60
    q[0, 5] *= 1e-3
    return K, V, q.astype(np.float16)


def test_edge_scale_bounds_hold():
    """The inputs reach the cases they are meant to (checked on the oracle's scales)."""
    for bits in (2, 4):
        K, V, q = edge_inputs(bits)
        oc = O.LayerCache(B, H, D, bits, G, D, R, 512)
        oc.prefill(K[:, :, :T0], V[:, :, :T0])
        Tq = oc.Tq
        ks = oc.k_scale[0, :, :Tq // G].astype(np.float64)
        vs = oc.v_scale[0, :, :Tq].astype(np.float64)
        assert ks[4].max() == 0 and vs[4].max() == 0
        assert 0 < ks[5].max() < 2.0 ** -14 and 0 < vs[5].max() < 2.0 ** -14
        qmax = np.abs(q[0, 5].astype(np.float64)).max() / math.sqrt(D) * math.log2(math.e)
        assert qmax * ks[5].max() < 2.0 ** -30
        assert ks[0].max() > 4e3 and vs[0].max() > 4e3     # near 65504 / (2^b - 1)


def check(got, ref, V, where):
    """R9 on every element; on head 5, whose values are multiples of 2^-24, also a
    bound relative to that head's largest value (R9's absolute term would accept any
    output there)."""
    assert_close(got, ref, where)
    scale = float(np.abs(V[0, 5].astype(np.float64)).max())
    err5 = np.abs(got[0, 5].astype(np.float64) - ref[0, 5])
    assert err5.max() <= 1e-4 * scale, f"{where}: subnormal head err {err5.max():.3e}"


@pytest.mark.gpu
@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("n_split", [0, 1, 3])
def test_decode_on_edge_caches(bits, n_split):
    from bit_quantization_amd import kivi as k
    K, V, q = edge_inputs(bits)
    w = W.Workload("edge", 91, 1, B, H, H, D, T0, bits, G, D, R, stream_steps=EXTRA)
    dims = dims_of(w, w.max_tokens())
    Kd, Vd = torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda()
    qd = torch.from_numpy(q).cuda()
    sm = 1 / math.sqrt(D)
    cache = gpu_prefill(w, dims, Kd, Vd, T0)
    out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
    ws = k.new_workspace(dims, T0 + EXTRA, n_split)
    k.kivi_decode_attn(dims, cache, 0, T0, qd, sm, out, ws, n_split=n_split)
    torch.cuda.synchronize()
    oc = O.LayerCache(B, H, D, bits, G, D, R, w.max_tokens())
    oc.prefill(K[:, :, :T0], V[:, :, :T0])
    check(out.cpu().numpy(), oc.attend(q, sm), V, f"decode bits={bits} n_split={n_split}")
    if n_split:
        return
    # fused append + decode: the first step flushes the full window
    for t in range(T0, T0 + 3):
        k.kivi_append_decode(dims, cache, 0, t, Kd[:, :, t].contiguous(), Vd[:, :, t].contiguous(),
                             qd, sm, out, ws)
        torch.cuda.synchronize()
        oc.append(K[:, :, t], V[:, :, t])
        check(out.cpu().numpy(), oc.attend(q, sm), V, f"append_decode bits={bits} T={t + 1}")
