"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test ties an oracle function to something other than itself: numbers printed
on the pages, hand-derived closed forms, exact rational arithmetic, brute force on
tiny inputs, a library routine (torch's scaled_dot_product_attention) or an
invariant the method guarantees.  They are chosen so that a dropped term, a wrong
sign or index, or a transposed operand in the oracle fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from tests.conftest import GOLDEN

F16, F32 = np.float16, np.float32


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------------
# Memory accounting
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("case", _load("kv_bytes.json")["cases"], ids=lambda c: c["cite"][:60])
def test_kv_bytes_match_page_numbers(case):
    n = O.kv_cache_bytes(case["layers"], case["batch"], case["tokens"], case["kv_heads"],
                         case["head_dim"], case["bytes_per_elem"])
    unit = {"GB": 1e9, "KB": 1e3, "GiB": 2.0 ** 30}[case["unit"]]
    assert abs(n / unit - case["printed"]) <= case["abs_tol"] + 1e-12


def test_kivi_bytes_codes_are_the_lower_bound():
    # 4.4 KV Cache quantization, section 1: the 2-bit figure counts codes only;
    # scale/zero and the residual come on top.
    acc = O.kivi_cache_bytes(32, 1, 32768, 8, 128, bits=2, group_k=32, group_v=128,
                             residual=128)
    lower = O.kv_cache_bytes(32, 1, 32768, 8, 128, 0.25)
    assert acc["codes"] < lower          # the last R tokens are fp16, not codes
    assert acc["total"] > lower
    # With no residual left behind (T a multiple of R plus the lazy window of R)
    Tq = O.quantized_len(32768, 128)
    assert acc["codes"] == O.kv_cache_bytes(32, 1, Tq, 8, 128, 0.25)
    assert acc["residual"] == O.kv_cache_bytes(32, 1, 128, 8, 128, 2)


def test_bytes_per_token_per_head_2bit_and_4bit():
    # Amortized bytes per cached token per KV head at d=128, G=32, G_v=128:
    # codes 2*d*b/8, K scale+zero 4*d/G, V scale+zero 4*d/G_v.
    for bits, expect in ((2, 84), (4, 148)):
        acc = O.kivi_cache_bytes(1, 1, 32 * 128 + 1, 1, 128, bits, 32, 128, 1 * 32)
        Tq = O.quantized_len(32 * 128 + 1, 32)
        per_tok = (acc["codes"] + acc["k_meta"] + acc["v_meta"]) / Tq
        assert per_tok == expect


# ----------------------------------------------------------------------------------
# Quantizer
# ----------------------------------------------------------------------------------

def _f16(vals):
    return np.array([float(v) for v in vals], F16)


@pytest.mark.parametrize("case", _load("quantizer_cases.json")["cases"], ids=lambda c: c["name"])
def test_quantizer_closed_forms(case):
    x = _f16(case["x"])
    codes, scale, zero = O.quantize_groups(x[None, :], case["bits"])
    assert codes[0].tolist() == case["codes"]
    if "scale_bits" in case:
        assert int(scale.view(np.uint16)[0]) == case["scale_bits"]
    else:
        assert float(scale[0]) == case["scale"]
    assert float(zero[0]) == case["zero"]
    if "zero_bits" in case:
        assert int(zero.view(np.uint16)[0]) == case["zero_bits"]
    assert int(scale.view(np.uint16)[0]) & 0x8000 == 0     # scale is never -0


def _random_groups(rng, n_groups, n, bits, kind):
    if kind == "normal":
        x = rng.standard_normal((n_groups, n)).astype(F32)
        x *= rng.choice([1e-3, 1.0, 50.0, 1000.0], size=(n_groups, 1)).astype(F32)
    elif kind == "tiny":     # ranges whose scale is a float16 subnormal or underflows
        x = (rng.standard_normal((n_groups, n)) * 1e-6).astype(F32)
        x += rng.choice([0.0, 1e-5, -3e-3], size=(n_groups, 1)).astype(F32)
    elif kind == "bits":     # arbitrary finite float16 bit patterns
        raw = rng.integers(0, 0x7C00, size=(n_groups, n), dtype=np.uint16)
        sign = rng.integers(0, 2, size=(n_groups, n), dtype=np.uint16) << 15
        return (raw | sign).view(F16)
    return x.astype(F16)


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("kind", ["normal", "tiny", "bits"])
def test_round_trip_error_within_half_step(bits, kind):
    """|x - x_hat| <= scale/2 (plus float32 rounding), the defining property of
    round-to-nearest on the min/max grid."""
    rng = np.random.default_rng(7 + bits)
    x = _random_groups(rng, 4000, 32, bits, kind)
    codes, scale, zero = O.quantize_groups(x, bits)
    xh = O.dequantize(codes, scale[:, None], zero[:, None]).astype(np.float64)
    xd = x.astype(np.float64)
    s = scale.astype(np.float64)[:, None]
    qmax = 2 ** bits - 1
    rng_ = xd.max(1, keepdims=True) - xd.min(1, keepdims=True)
    ulp = 2.0 ** -23 * (np.abs(xd) + np.abs(xh) + rng_)
    normal = s >= 2.0 ** -14
    bound = np.where(normal, s / 2, s / 2 + qmax * 2.0 ** -25)
    bound = np.where(s == 0, rng_, bound)       # degenerate groups: error <= range
    err = np.abs(xd - xh)
    assert np.all(err <= bound + 4 * ulp)
    assert np.all(codes <= qmax)


@pytest.mark.parametrize("bits", [2, 4])
def test_min_maps_to_zero_and_max_to_top_code(bits):
    rng = np.random.default_rng(11)
    x = _random_groups(rng, 3000, 32, bits, "normal")
    codes, scale, zero = O.quantize_groups(x, bits)
    s = scale.astype(np.float64)
    ok = s >= 2.0 ** -14
    imin = np.argmin(x.astype(F32), axis=1)
    imax = np.argmax(x.astype(F32), axis=1)
    rows = np.arange(len(x))
    assert np.all(codes[rows, imin][ok] == 0)
    assert np.all(codes[rows, imax][ok] == 2 ** bits - 1)
    assert np.all(zero.astype(F32) == x.astype(F32).min(1))


def _nearest_even(q: Fraction) -> int:
    lo = math.floor(q)
    d = q - lo
    if d < Fraction(1, 2):
        return lo
    if d > Fraction(1, 2):
        return lo + 1
    return lo if lo % 2 == 0 else lo + 1


@pytest.mark.parametrize("bits", [2, 4])
def test_codes_are_nearest_grid_points_exact_arithmetic(bits):
    """Brute force with exact rationals: each code is the grid point k*scale + min
    nearest to x (ties to even k), except where float32 rounding of (x - min)/scale
    lands exactly on a half-integer the exact quotient is not on."""
    rng = np.random.default_rng(5)
    x = _random_groups(rng, 600, 8, bits, "normal")
    codes, scale, zero = O.quantize_groups(x, bits)
    qmax = 2 ** bits - 1
    near_ties = 0
    for i in range(len(x)):
        s = Fraction(float(scale[i]))
        mn = Fraction(float(zero[i]))
        for j in range(x.shape[1]):
            xv = Fraction(float(x[i, j]))
            if s == 0:
                assert codes[i, j] == 0
                continue
            qe = (xv - mn) / s
            k = min(max(_nearest_even(qe), 0), qmax)
            if codes[i, j] != k:
                # only allowed when the exact quotient is within float32 rounding of
                # a tie and the codes differ by one
                frac = qe - math.floor(qe)
                assert abs(frac - Fraction(1, 2)) < Fraction(1, 2 ** 20)
                assert abs(int(codes[i, j]) - k) == 1
                near_ties += 1
    assert near_ties <= 2


def test_constant_and_degenerate_groups_dequantize_exactly():
    x = np.array([[1.5] * 32, [-7.0] * 32, [0.0] * 32, [65504.0] * 32], F16)
    for bits in (2, 4):
        codes, scale, zero = O.quantize_groups(x, bits)
        assert np.all(codes == 0) and np.all(scale == 0)
        xh = O.dequantize(codes, scale[:, None], zero[:, None])
        assert np.array_equal(xh, x.astype(F32))


def test_full_float16_range_does_not_overflow():
    x = np.array([[-65504.0, 65504.0, 0.0, 1.0]], F16)
    for bits in (2, 4):
        codes, scale, zero = O.quantize_groups(x, bits)
        assert np.isfinite(float(scale[0])) and codes[0, 0] == 0
        assert codes[0, 1] == 2 ** bits - 1


# ----------------------------------------------------------------------------------
# Grouping axes
# ----------------------------------------------------------------------------------

def test_key_groups_run_over_tokens_of_one_channel_bruteforce():
    rng = np.random.default_rng(2)
    T, d, G, bits = 64, 8, 16, 2
    K = (rng.standard_normal((T, d)) * 3).astype(F16)
    codes, scale, zero = O.quantize_keys(K, G, bits)
    assert scale.shape == (T // G, d)
    for g in range(T // G):
        for c in range(d):
            col = [float(K[t, c]) for t in range(g * G, (g + 1) * G)]
            mn, mx = min(col), max(col)
            assert float(zero[g, c]) == mn + 0.0
            assert scale[g, c] == np.float16(np.float32(np.float32(mx) - np.float32(mn)) / F32(3))


def test_value_groups_run_over_channels_of_one_token_bruteforce():
    rng = np.random.default_rng(3)
    T, d, Gv, bits = 5, 16, 8, 4
    V = (rng.standard_normal((T, d)) * 3).astype(F16)
    codes, scale, zero = O.quantize_values(V, Gv, bits)
    assert scale.shape == (T, d // Gv)
    for t in range(T):
        for j in range(d // Gv):
            row = [float(V[t, c]) for c in range(j * Gv, (j + 1) * Gv)]
            mn, mx = min(row), max(row)
            assert float(zero[t, j]) == mn + 0.0
            assert scale[t, j] == np.float16(np.float32(np.float32(mx) - np.float32(mn)) / F32(15))


def test_per_channel_keys_contain_outlier_channels():
    """'KV Cache Quantization (KIVI & FP4)' section 6.5 and 'KIVI: A Tuning-Free ...',
    'Keys and values are not the same tensor': with a few Key channels tens of times
    larger than the rest, per-token grouping inflates the step of every normal
    channel, while per-channel grouping keeps normal channels fine.  A transposed
    grouping in the oracle fails this."""
    rng = np.random.default_rng(4)
    T, d, G = 256, 128, 32
    K = rng.standard_normal((T, d)).astype(F32)
    K[:, [3, 40, 77, 100]] *= 50
    K = K.astype(F16)
    normal = np.setdiff1d(np.arange(d), [3, 40, 77, 100])
    kc, ks, kz = O.quantize_keys(K, G, 2)
    per_channel = O.dequantize_keys(kc, ks, kz, G)
    vc, vs, vz = O.quantize_values(K, d, 2)        # the same data grouped per token
    per_token = O.dequantize_values(vc, vs, vz, d)
    e_ch = np.abs(per_channel - K.astype(F32))[:, normal].mean()
    e_tok = np.abs(per_token - K.astype(F32))[:, normal].mean()
    assert e_ch * 10 < e_tok


def test_per_token_values_contain_outlier_tokens():
    """'09 — KV Cache Quantization', 'The structural fact...': Value outliers are
    whole tokens; per-token grouping isolates them."""
    rng = np.random.default_rng(5)
    T, d = 64, 128
    V = rng.standard_normal((T, d)).astype(F32)
    V[[0, 17, 40]] *= 100
    V = V.astype(F16)
    normal = np.setdiff1d(np.arange(T), [0, 17, 40])
    vc, vs, vz = O.quantize_values(V, d, 2)
    per_token = O.dequantize_values(vc, vs, vz, d)
    kc, ks, kz = O.quantize_keys(V, 32, 2)         # the same data grouped per channel
    per_channel = O.dequantize_keys(kc, ks, kz, 32)
    e_tok = np.abs(per_token - V.astype(F32))[normal].mean()
    e_ch = np.abs(per_channel - V.astype(F32))[normal].mean()
    assert e_tok * 5 < e_ch


# ----------------------------------------------------------------------------------
# Packing
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("case", _load("packing_cases.json")["cases"])
def test_packing_hand_vectors(case):
    c = np.array(case["codes"], np.uint8)[None]
    packed = O.pack_words(c, case["bits"])
    assert packed[0].tolist() == case["bytes"]
    assert np.array_equal(O.unpack_words(packed, case["bits"]), c)


@pytest.mark.parametrize("bits", [2, 4])
def test_key_and_value_layouts_place_each_code_where_stated(bits):
    rng = np.random.default_rng(6)
    T, d = 48, 32
    codes = rng.integers(0, 2 ** bits, size=(T, d), dtype=np.uint8)
    n = 32 // bits                                 # codes per 32-bit word

    def code_at(row, j):
        # code j of a packed run: word j // n, byte 4*(j // n) + (j % n) % 4,
        # bit offset bits * ((j % n) // 4)
        e = j % n
        byte = int(row[4 * (j // n) + e % 4])
        return (byte >> (bits * (e // 4))) & (2 ** bits - 1)

    pk = O.pack_keys(codes, bits)
    pv = O.pack_values(codes, bits)
    assert pk.shape == (T, d * bits // 8) and pv.shape == (T // 16, d, 16 * bits // 8)
    for t in range(T):
        for c in range(d):
            assert code_at(pk[t], c) == codes[t, c]
            assert code_at(pv[t // 16, c], t % 16) == codes[t, c]
    assert np.array_equal(O.unpack_keys(pk, bits), codes)
    assert np.array_equal(O.unpack_values(pv, bits), codes)


# ----------------------------------------------------------------------------------
# Residual window and streaming
# ----------------------------------------------------------------------------------

def test_residual_split_table():
    R = 32
    assert [O.residual_len(T, R) for T in (0, 1, 31, 32, 33, 64, 65, 256)] == \
        [0, 1, 31, 32, 1, 32, 1, 32]
    assert O.quantized_len(256, 32) == 224          # 256 tokens, R=32: 224 + 32 fp16
    assert O.quantized_len(32768, 128) == 32640
    assert O.quantized_len(131072, 128) == 130944
    assert O.quantized_len(1048576, 128) == 1048448
    # 256 streamed steps after a 32768 prefill flush at steps 1 and 129 only
    flushes = [s for s in range(1, 257) if O.residual_len(32768 + s - 1, 128) == 128]
    assert flushes == [1, 129]


def _cache(B, H, d, bits, G, Gv, R, Tmax):
    return O.LayerCache(B, H, d, bits, G, Gv, R, Tmax)


@pytest.mark.parametrize("bits,G,Gv,R", [(2, 32, 128, 32), (4, 32, 64, 64), (2, 16, 32, 48)])
def test_prefill_equals_streaming_appends(bits, G, Gv, R):
    """Quantization is group-local, so prefill(T) and T single appends reach the same
    bytes ('KIVI: A Tuning-Free ...', 'The streaming complication')."""
    rng = np.random.default_rng(8)
    B, H, d, T = 2, 2, 128, 3 * R + 5
    K = (rng.standard_normal((B, H, T, d)) * 2).astype(F16)
    V = (rng.standard_normal((B, H, T, d)) * 2).astype(F16)
    Tmax = 4 * R + 16 * 4
    Tmax = (Tmax + 47) // 48 * 48 if R == 48 else Tmax
    for Tp in (0, 1, R - 1, R, R + 1, 2 * R, T):
        a = _cache(B, H, d, bits, G, Gv, R, Tmax)
        a.prefill(K[:, :, :Tp], V[:, :, :Tp])
        for t in range(Tp, T):
            a.append(K[:, :, t], V[:, :, t])
        b = _cache(B, H, d, bits, G, Gv, R, Tmax)
        b.prefill(K, V)
        for name in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero"):
            assert np.array_equal(getattr(a, name).view(np.uint8), getattr(b, name).view(np.uint8)), name
        r = O.residual_len(T, R)
        assert np.array_equal(a.k_resid[:, :, :r], b.k_resid[:, :, :r])
        assert np.array_equal(a.v_resid[:, :, :r], b.v_resid[:, :, :r])


def test_residual_holds_the_most_recent_tokens_in_fp16():
    rng = np.random.default_rng(9)
    B, H, d, R = 1, 1, 128, 32
    K = rng.standard_normal((B, H, 256, d)).astype(F16)
    c = _cache(B, H, d, 2, 32, 128, R, 320)
    c.prefill(K, K)
    Kh, Vh = c.dequantized()
    assert np.array_equal(Kh[:, :, 224:], K[:, :, 224:].astype(F32))   # exact fp16 tail
    assert not np.array_equal(Kh[:, :, :224], K[:, :, :224].astype(F32))


# ----------------------------------------------------------------------------------
# Attention
# ----------------------------------------------------------------------------------

def _brute_attention(q, K, V, sm):
    """Scalar loops with math.exp: no numpy reductions, no shortcuts."""
    T, d = len(K), len(q)
    z = []
    for t in range(T):
        acc = 0.0
        for c in range(d):
            acc += float(q[c]) * float(K[t][c])
        z.append(float(np.float32(sm)) * acc)
    m = max(z)
    w = [math.exp(v - m) for v in z]
    s = sum(w)
    return [sum(w[t] * float(V[t][c]) for t in range(T)) / s for c in range(d)]


def test_attention_matches_scalar_bruteforce():
    rng = np.random.default_rng(10)
    T, d = 37, 16
    q = rng.standard_normal((1, d)).astype(F16)
    K = (rng.standard_normal((T, d)) * 2).astype(F32)
    V = (rng.standard_normal((T, d)) * 2).astype(F32)
    sm = 1 / math.sqrt(d)
    got = O.attention_fp64(q, K, V, sm)[0]
    ref = _brute_attention(q[0], K, V, sm)
    assert np.allclose(got, ref, rtol=1e-6, atol=1e-6)


def test_quantized_cache_attention_matches_bruteforce_on_codes():
    """End-to-end: cache of 3 groups + ragged residual, brute force over the
    dequantized rows computed by hand from codes, scale and zero."""
    rng = np.random.default_rng(12)
    B, H, Hq, d, G, R, bits = 1, 1, 2, 32, 16, 16, 2
    T = 3 * 16 + 5
    K = (rng.standard_normal((B, H, T, d)) * 2).astype(F16)
    V = (rng.standard_normal((B, H, T, d)) * 2).astype(F16)
    c = _cache(B, H, d, bits, G, d, R, 96)
    c.prefill(K, V)
    q = rng.standard_normal((B, Hq, d)).astype(F16)
    got = c.attend(q, 0.3)
    Tq = O.quantized_len(T, R)
    kc, vc = c.quantized_codes()
    rowsK, rowsV = [], []
    for t in range(T):
        if t < Tq:
            g = t // G
            rowsK.append([float(kc[0, 0, t, ch]) * float(c.k_scale[0, 0, g, ch])
                          + float(c.k_zero[0, 0, g, ch]) for ch in range(d)])
            rowsV.append([float(vc[0, 0, t, ch]) * float(c.v_scale[0, 0, t, 0])
                          + float(c.v_zero[0, 0, t, 0]) for ch in range(d)])
        else:
            rowsK.append([float(x) for x in c.k_resid[0, 0, t - Tq]])
            rowsV.append([float(x) for x in c.v_resid[0, 0, t - Tq]])
    for j in range(Hq):
        ref = _brute_attention(q[0, j], rowsK, rowsV, 0.3)
        assert np.allclose(got[0, j], ref, rtol=1e-5, atol=1e-5)


def test_unquantized_window_equals_torch_sdpa():
    """T <= R: nothing is quantized, so decode attention is plain SDPA (library)."""
    import torch
    rng = np.random.default_rng(13)
    B, H, Hq, d, R = 2, 2, 8, 64, 32
    T = 29
    K = rng.standard_normal((B, H, T, d)).astype(F16)
    V = rng.standard_normal((B, H, T, d)).astype(F16)
    q = rng.standard_normal((B, Hq, d)).astype(F16)
    c = _cache(B, H, d, 2, 16, 64, R, 64)
    c.prefill(K, V)
    got = c.attend(q, 1 / math.sqrt(d))
    g = Hq // H
    Kr = torch.from_numpy(np.repeat(K.astype(np.float64), g, axis=1))
    Vr = torch.from_numpy(np.repeat(V.astype(np.float64), g, axis=1))
    qt = torch.from_numpy(q.astype(np.float64))[:, :, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, Kr, Vr, scale=float(np.float32(1 / math.sqrt(d))))[:, :, 0, :].numpy()
    assert np.allclose(got, ref, rtol=1e-6, atol=1e-6)


def test_on_grid_data_is_reproduced_exactly():
    """If every K group and V token already lies on its min/max grid, quantization
    is lossless and the quantized attention equals unquantized attention."""
    rng = np.random.default_rng(14)
    B, H, d, G, R, bits = 1, 2, 32, 16, 16, 2
    T = 4 * 16 + 3
    Tq = O.quantized_len(T, R)
    K = np.zeros((B, H, T, d), F32)
    V = np.zeros((B, H, T, d), F32)
    for h in range(H):
        for g in range(Tq // G):
            for ch in range(d):
                s, mn = 0.25 * rng.integers(1, 8), 0.5 * rng.integers(-8, 8)
                codes = rng.integers(0, 4, size=G)
                codes[0], codes[1] = 0, 3
                K[0, h, g * G:(g + 1) * G, ch] = codes * s + mn
        for t in range(Tq):
            s, mn = 0.125 * rng.integers(1, 8), 0.5 * rng.integers(-8, 8)
            codes = rng.integers(0, 4, size=d)
            codes[0], codes[1] = 0, 3
            V[0, h, t] = codes * s + mn
    K[:, :, Tq:] = rng.standard_normal((B, H, T - Tq, d))
    V[:, :, Tq:] = rng.standard_normal((B, H, T - Tq, d))
    K, V = K.astype(F16), V.astype(F16)
    c = _cache(B, H, d, bits, G, d, R, 96)
    c.prefill(K, V)
    Kh, Vh = c.dequantized()
    assert np.array_equal(Kh, K.astype(F32)) and np.array_equal(Vh, V.astype(F32))
    q = rng.standard_normal((B, 4, d)).astype(F16)
    got = c.attend(q, 0.2)
    ref = O.gqa_attention_fp64(q, K.astype(F32), V.astype(F32), 0.2)
    assert np.array_equal(got, ref)


def test_zero_query_averages_the_values():
    rng = np.random.default_rng(15)
    B, H, d = 1, 1, 128
    K = (rng.standard_normal((B, H, 100, d)) * 5).astype(F16)
    V = (rng.standard_normal((B, H, 100, d)) * 5).astype(F16)
    c = _cache(B, H, d, 4, 32, 128, 32, 128)
    c.prefill(K, V)
    got = c.attend(np.zeros((B, 1, d), F16), 0.1)
    _, Vh = c.dequantized()
    assert np.allclose(got[0, 0], Vh[0, 0].astype(np.float64).mean(0), rtol=1e-6, atol=1e-6)


def test_gqa_head_mapping_is_consecutive():
    """Query head j reads KV head j // g: equal to MHA with each KV head repeated."""
    rng = np.random.default_rng(16)
    B, H, g, d, T = 2, 3, 4, 32, 40
    K = rng.standard_normal((B, H, T, d)).astype(F32)
    V = rng.standard_normal((B, H, T, d)).astype(F32)
    q = rng.standard_normal((B, H * g, d)).astype(F16)
    got = O.gqa_attention_fp64(q, K, V, 0.3)
    ref = O.gqa_attention_fp64(q, np.repeat(K, g, axis=1), np.repeat(V, g, axis=1), 0.3)
    assert np.array_equal(got, ref)
    # and a different KV head gives a different answer (the mapping matters)
    other = O.attention_fp64(q[0, :1], K[0, 1], V[0, 1], 0.3)
    assert not np.allclose(got[0, 0], other[0])


def test_shift_of_logits_leaves_attention_unchanged():
    """Adding c*q/|q|^2 * (1/sm) to every key shifts all logits by c: softmax is
    invariant (checks that the max subtraction is applied consistently)."""
    rng = np.random.default_rng(17)
    d, T = 16, 50
    q = rng.standard_normal((1, d)).astype(F32)
    K = rng.standard_normal((T, d)).astype(np.float64)
    V = rng.standard_normal((T, d)).astype(np.float64)
    sm = 0.25
    a = O.attention_fp64(q, K, V, sm)
    shift = q[0].astype(np.float64) / float(q[0].astype(np.float64) @ q[0]) * (30.0 / float(np.float32(sm)))
    b = O.attention_fp64(q, K + shift, V, sm)
    assert np.allclose(a, b, rtol=1e-9, atol=1e-9)


# ---- sink tokens (reading R15) ---------------------------------------------------------

def _sink_inputs(T, seed):
    rng = np.random.default_rng(seed)
    K = (rng.standard_normal((2, 2, T, 128)) * 2).astype(np.float16)
    V = (rng.standard_normal((2, 2, T, 128)) * 2).astype(np.float16)
    K[:, :, :, 5] *= 40
    return K, V


def test_sink_rows_are_the_inputs_exactly():
    K, V = _sink_inputs(300, 1)
    c = O.LayerCache(2, 2, 128, 2, 32, 128, 64, 512, sink=4)
    c.prefill(K, V)
    Kh, Vh = c.dequantized()
    assert np.array_equal(Kh[:, :, :4], K[:, :, :4].astype(np.float32))
    assert np.array_equal(Vh[:, :, :4], V[:, :, :4].astype(np.float32))
    assert Kh.shape[2] == 300


def test_sink_covering_every_token_is_plain_sdpa():
    import torch
    K, V = _sink_inputs(40, 2)
    c = O.LayerCache(2, 2, 128, 2, 32, 128, 32, 128, sink=64)
    c.prefill(K, V)
    q = np.random.default_rng(3).standard_normal((2, 4, 128)).astype(np.float16)
    got = c.attend(q, 0.088)
    for b in range(2):
        for j in range(4):
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[b, j:j + 1].astype(np.float64))[None],
                torch.from_numpy(K[b, j // 2].astype(np.float64))[None],
                torch.from_numpy(V[b, j // 2].astype(np.float64))[None],
                scale=float(np.float32(0.088)))
            assert np.allclose(got[b, j], ref[0, 0].numpy(), rtol=1e-6, atol=1e-6)


def test_tokens_after_the_sink_follow_the_plain_method_from_s():
    S, T = 7, 400
    K, V = _sink_inputs(T, 4)
    a = O.LayerCache(2, 2, 128, 4, 32, 64, 64, 512, sink=S)
    a.prefill(K, V)
    b = O.LayerCache(2, 2, 128, 4, 32, 64, 64, 512)
    b.prefill(K[:, :, S:], V[:, :, S:])
    Ka, Va = a.dequantized()
    Kb, Vb = b.dequantized()
    assert np.array_equal(Ka[:, :, S:], Kb) and np.array_equal(Va[:, :, S:], Vb)
    assert np.array_equal(a.k_codes, b.k_codes) and np.array_equal(a.v_codes, b.v_codes)


@pytest.mark.parametrize("S,T0", [(4, 0), (4, 2), (4, 4), (9, 30), (64, 50)])
def test_sink_prefill_equals_appends(S, T0):
    T = S + 2 * 64 + 11
    K, V = _sink_inputs(T, 5 + S)
    a = O.LayerCache(2, 2, 128, 2, 32, 128, 64, 512, sink=S)
    a.prefill(K, V)
    b = O.LayerCache(2, 2, 128, 2, 32, 128, 64, 512, sink=S)
    b.prefill(K[:, :, :T0], V[:, :, :T0])
    for t in range(T0, T):
        b.append(K[:, :, t], V[:, :, t])
    for name in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero", "k_sink",
                 "v_sink"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
    r = O.residual_len(T - S, 64)
    assert np.array_equal(a.k_resid[:, :, :r], b.k_resid[:, :, :r])


# ---- group-wise aging of the window (reading R16) --------------------------------------

def test_grouped_window_length_table():
    # R = 64, G = 16: the window fills to 64, then each arriving token at a full
    # window sends one group of 16 out: 65 -> 49, 80 -> 64, 81 -> 49; 200 -> 48 + 8
    table = {0: 0, 1: 1, 63: 63, 64: 64, 65: 49, 66: 50, 79: 63, 80: 64, 81: 49, 200: 56}
    for T, r in table.items():
        assert O.residual_len_grouped(T, 64, 16) == r, T
    for T in range(0, 300):
        assert O.residual_len_grouped(T, 32, 32) == O.residual_len(T, 32)
        if T > 64:
            r = O.residual_len_grouped(T, 64, 16)
            assert 49 <= r <= 64 and (T - r) % 16 == 0


def _aging_stream(R, G, S, T, seed, bits=2, Gv=128):
    K, V = _sink_inputs(T, seed)
    c = O.LayerCache(2, 2, 128, bits, G, Gv, R, 512, sink=S, aging="group")
    return K, V, c


def test_grouped_aging_flushes_one_group_at_a_time():
    R, G, T = 64, 16, 170
    K, V, c = _aging_stream(R, G, 0, T, 21)
    grew = []
    for t in range(T):
        before = c.Tq
        c.append(K[:, :, t], V[:, :, t])
        if c.Tq != before:
            grew.append((t, c.Tq - before))
        r = c.Tk - c.Tq
        # the window is the r most recent tokens, exactly, oldest first
        assert np.array_equal(c.k_resid[:, :, :r], K[:, :, t + 1 - r:t + 1])
        assert np.array_equal(c.v_resid[:, :, :r], V[:, :, t + 1 - r:t + 1])
    assert grew == [(t, 16) for t in range(64, T, 16)]


@pytest.mark.parametrize("R,G,S,T0,bits", [(64, 16, 0, 0, 2), (64, 32, 0, 40, 4),
                                           (128, 32, 5, 3, 2), (96, 32, 0, 200, 4)])
def test_grouped_aging_prefill_equals_appends(R, G, S, T0, bits):
    T = S + 3 * R + 13
    K, V, a = _aging_stream(R, G, S, T, 30 + G, bits)
    a.prefill(K, V)
    _, _, b = _aging_stream(R, G, S, T, 30 + G, bits)
    b.prefill(K[:, :, :T0], V[:, :, :T0])
    for t in range(T0, T):
        b.append(K[:, :, t], V[:, :, t])
    for name in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero", "k_sink",
                 "v_sink"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
    r = a.Tk - a.Tq
    assert r == b.Tk - b.Tq == O.residual_len_grouped(T - S, R, G)
    assert np.array_equal(a.k_resid[:, :, :r], b.k_resid[:, :, :r])
    assert np.array_equal(a.v_resid[:, :, :r], b.v_resid[:, :, :r])


def test_grouped_aging_with_one_group_windows_is_the_window_rule():
    T = 3 * 32 + 9
    K, V = _sink_inputs(T, 40)
    a = O.LayerCache(2, 2, 128, 2, 32, 128, 32, 256, aging="group")
    b = O.LayerCache(2, 2, 128, 2, 32, 128, 32, 256)
    for t in range(T):
        a.append(K[:, :, t], V[:, :, t])
        b.append(K[:, :, t], V[:, :, t])
    for name in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero", "k_resid",
                 "v_resid"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name


@pytest.mark.parametrize("T", [64, 65, 100, 129, 200, 257])
def test_grouped_history_matches_window_history_on_the_common_prefix(T):
    # groups are quantized on their own, so the history of either rule holds the same
    # codes, scales and zeros for every token both have quantized
    K, V = _sink_inputs(T, 50)
    a = O.LayerCache(2, 2, 128, 4, 16, 64, 64, 512, aging="group")
    b = O.LayerCache(2, 2, 128, 4, 16, 64, 64, 512)
    a.prefill(K, V)
    b.prefill(K, V)
    n = min(a.Tq, b.Tq)
    assert a.Tq == T - O.residual_len_grouped(T, 64, 16) and b.Tq == O.quantized_len(T, 64)
    assert np.array_equal(a.k_codes[:, :, :n], b.k_codes[:, :, :n])
    assert np.array_equal(a.k_scale[:, :, :n // 16], b.k_scale[:, :, :n // 16])
    assert np.array_equal(a.k_zero[:, :, :n // 16], b.k_zero[:, :, :n // 16])
    assert np.array_equal(a.v_codes[:, :, :n // 16], b.v_codes[:, :, :n // 16])
    assert np.array_equal(a.v_scale[:, :, :n], b.v_scale[:, :, :n])
    Kh, Vh = a.dequantized()
    r = T - a.Tq
    assert np.array_equal(Kh[:, :, T - r:], K[:, :, T - r:].astype(np.float32))
    assert np.array_equal(Vh[:, :, T - r:], V[:, :, T - r:].astype(np.float32))
