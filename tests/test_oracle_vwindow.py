"""Pins of the oracle's per-token Value window (reading R21, "4.4 KV Cache
quantization" §3.2): Values leave a window of exactly R tokens one at a time, each
quantized on its own as it leaves; Keys keep their group rule.  Checked against
the plain window rule, per-token definitions, hand-computed dequantization with
scalar brute-force attention, torch's SDPA on lossless data, and the
prefill/append equivalence.  CPU only."""
import math

import numpy as np
import pytest

import oracle as O

F16, F32 = np.float16, np.float32


def _pair(B, H, d, bits, G, R, Tmax, S=0, aging="window"):
    tok = O.LayerCache(B, H, d, bits, G, d, R, Tmax, sink=S, aging=aging, v_window="token")
    ref = O.LayerCache(B, H, d, bits, G, d, R, Tmax, sink=S, aging=aging)
    return tok, ref


@pytest.mark.parametrize("R,G,S,aging", [(32, 32, 0, "window"), (32, 16, 0, "group"),
                                         (48, 16, 3, "window"), (64, 32, 5, "group")])
def test_token_window_state_through_a_stream(R, G, S, aging):
    """At every step: T_qv = max(0, T_k - R); the Value window is the most recent
    min(T_k, R) inputs bit for bit; the Key side equals the plain cache's; the
    quantized Values equal one-shot per-token quantization of those inputs."""
    rng = np.random.default_rng(R + G + S)
    B, H, d, bits = 1, 2, 32, 2
    T = S + 4 * R + 7
    K = (rng.standard_normal((B, H, T, d)) * 3).astype(F16)
    V = (rng.standard_normal((B, H, T, d)) * 3).astype(F16)
    Tmax = ((T + 64) // 64 + 1) * 64
    tok, ref = _pair(B, H, d, bits, G, R, Tmax, S, aging)
    middle_seen = False
    for t in range(T):
        tok.append(K[:, :, t], V[:, :, t])
        ref.append(K[:, :, t], V[:, :, t])
        Tk = max(0, t + 1 - S)
        Tqv = max(0, Tk - R)
        assert tok.Tqv == Tqv and tok.Tq == ref.Tq
        nv = Tk - Tqv
        assert nv == min(Tk, R)
        assert np.array_equal(tok.v_resid[:, :, :nv], V[:, :, S + Tqv:S + Tk])
        r = Tk - ref.Tq
        for name in ("k_codes", "k_scale", "k_zero"):
            assert np.array_equal(getattr(tok, name), getattr(ref, name)), (t, name)
        assert np.array_equal(tok.k_resid[:, :, :r], ref.k_resid[:, :, :r])
        if Tqv:
            vc, vs, vz = O.quantize_values(V[:, :, S:S + Tqv], d, bits)
            assert np.array_equal(tok.v_scale[:, :, :Tqv].view(np.int16), vs.view(np.int16))
            assert np.array_equal(tok.v_zero[:, :, :Tqv].view(np.int16), vz.view(np.int16))
            assert np.array_equal(tok.quantized_codes()[1], vc)
        middle_seen |= Tqv < tok.Tq
    # tokens whose Key is quantized while their Value is float16 occur (R21)
    assert middle_seen


@pytest.mark.parametrize("R,G,S,aging,T0", [(32, 32, 0, "window", 20), (32, 32, 0, "window", 33),
                                            (32, 16, 2, "group", 31), (48, 16, 0, "window", 160)])
def test_token_window_prefill_equals_appends(R, G, S, aging, T0):
    rng = np.random.default_rng(T0)
    B, H, d, bits = 2, 1, 32, 4
    T = T0 + 3 * R + 5
    K = rng.standard_normal((B, H, T, d)).astype(F16)
    V = rng.standard_normal((B, H, T, d)).astype(F16)
    Tmax = ((T + 64) // 64 + 1) * 64
    a = O.LayerCache(B, H, d, bits, G, d, R, Tmax, sink=S, aging=aging, v_window="token")
    a.prefill(K[:, :, :T0], V[:, :, :T0])
    for t in range(T0, T):
        a.append(K[:, :, t], V[:, :, t])
    b = O.LayerCache(B, H, d, bits, G, d, R, Tmax, sink=S, aging=aging, v_window="token")
    b.prefill(K, V)
    for name in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero"):
        x, y = getattr(a, name), getattr(b, name)
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), name
    r, rv = a.Tk - a.Tq, a.Tk - a.Tqv
    assert np.array_equal(a.k_resid[:, :, :r], b.k_resid[:, :, :r])
    assert np.array_equal(a.v_resid[:, :, :rv], b.v_resid[:, :, :rv])


def _brute_attention(q, K, V, sm):
    z = []
    for t in range(len(K)):
        z.append(float(np.float32(sm)) * sum(float(q[c]) * float(K[t][c]) for c in range(len(q))))
    m = max(z)
    w = [math.exp(v - m) for v in z]
    s = sum(w)
    return [sum(w[t] * float(V[t][c]) for t in range(len(K))) / s for c in range(len(q))]


def test_token_window_attention_matches_bruteforce_on_codes():
    """Rows rebuilt by hand: Keys from codes below T_q, Values from codes below
    T_qv (the middle tokens use their float16 Values), raw float16 above."""
    rng = np.random.default_rng(21)
    B, H, Hq, d, G, R, bits = 1, 1, 2, 32, 16, 32, 2
    T = 3 * 32 + 9          # Keys: window of 9, T_q = 96; Values: T_qv = T - R = 73
    K = (rng.standard_normal((B, H, T, d)) * 2).astype(F16)
    V = (rng.standard_normal((B, H, T, d)) * 2).astype(F16)
    c = O.LayerCache(B, H, d, bits, G, d, R, 128, v_window="token")
    c.prefill(K, V)
    Tq, Tqv = c.Tq, c.Tqv
    assert (Tq, Tqv) == (96, T - R) and Tqv < Tq
    kc, vc = c.quantized_codes()
    rowsK, rowsV = [], []
    for t in range(T):
        if t < Tq:
            g = t // G
            rowsK.append([float(kc[0, 0, t, ch]) * float(c.k_scale[0, 0, g, ch])
                          + float(c.k_zero[0, 0, g, ch]) for ch in range(d)])
        else:
            rowsK.append([float(x) for x in K[0, 0, t]])
        if t < Tqv:
            rowsV.append([float(vc[0, 0, t, ch]) * float(c.v_scale[0, 0, t, 0])
                          + float(c.v_zero[0, 0, t, 0]) for ch in range(d)])
        else:
            rowsV.append([float(x) for x in V[0, 0, t]])
    q = rng.standard_normal((B, Hq, d)).astype(F16)
    got = c.attend(q, 0.3)
    for j in range(Hq):
        assert np.allclose(got[0, j], _brute_attention(q[0, j], rowsK, rowsV, 0.3),
                           rtol=1e-5, atol=1e-5)


def test_token_window_on_grid_values_give_unquantized_attention():
    """Every Key group and Value token on its min/max grid: quantization is lossless
    and attention equals torch's float64 SDPA of the raw inputs."""
    import torch
    rng = np.random.default_rng(22)
    B, H, Hq, d, G, R, bits = 1, 1, 4, 32, 16, 32, 2
    T = 4 * 32 + 5
    K = np.zeros((B, H, T, d), F32)
    V = np.zeros((B, H, T, d), F32)
    for g in range(T // G):
        for ch in range(d):
            s, mn = 0.25 * rng.integers(1, 8), 0.5 * rng.integers(-8, 8)
            codes = rng.integers(0, 4, size=G)
            codes[0], codes[1] = 0, 3
            K[0, 0, g * G:(g + 1) * G, ch] = codes * s + mn
    K[0, 0, (T // G) * G:] = rng.standard_normal((T - (T // G) * G, d))
    for t in range(T):
        s, mn = 0.125 * rng.integers(1, 8), 0.5 * rng.integers(-8, 8)
        codes = rng.integers(0, 4, size=d)
        codes[0], codes[1] = 0, 3
        V[0, 0, t] = codes * s + mn
    K, V = K.astype(F16), V.astype(F16)
    c = O.LayerCache(B, H, d, bits, G, d, R, 160, v_window="token")
    for t in range(T):
        c.append(K[:, :, t], V[:, :, t])
    Kh, Vh = c.dequantized()
    assert np.array_equal(Kh, K.astype(F32)) and np.array_equal(Vh, V.astype(F32))
    q = rng.standard_normal((B, Hq, d)).astype(F16)
    got = c.attend(q, 0.2)
    Kr = torch.from_numpy(np.repeat(K.astype(np.float64), Hq, axis=1))
    Vr = torch.from_numpy(np.repeat(V.astype(np.float64), Hq, axis=1))
    qt = torch.from_numpy(q.astype(np.float64))[:, :, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, Kr, Vr, scale=float(np.float32(0.2)))[:, :, 0, :].numpy()
    assert np.allclose(got, ref, rtol=1e-6, atol=1e-6)


def test_token_window_short_sequences_are_plain_sdpa():
    """T_k <= R: no Value is quantized and, with T_k <= r, no Key either."""
    rng = np.random.default_rng(23)
    B, H, d, R = 1, 2, 32, 32
    T = 20
    K = rng.standard_normal((B, H, T, d)).astype(F16)
    V = rng.standard_normal((B, H, T, d)).astype(F16)
    c = O.LayerCache(B, H, d, 2, 16, d, R, 64, v_window="token")
    c.prefill(K, V)
    assert c.Tq == 0 and c.Tqv == 0
    Kh, Vh = c.dequantized()
    assert np.array_equal(Kh, K.astype(F32)) and np.array_equal(Vh, V.astype(F32))
