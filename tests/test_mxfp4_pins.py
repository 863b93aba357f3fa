"""Pins of the MXFP4 oracle (oracle/mxfp4_ref.py) against what the format definitions
and independent computations fix: the E2M1 code values, hand-derived roundings (every
tie, saturation, signs), brute-force nearest codes, the OCP block-scale rule on
closed-form blocks, the storage layout, and attention that reduces to plain SDPA when
the data lies on the MXFP4 grid."""
import math

import numpy as np
import pytest

import oracle as O

torch = pytest.importorskip("torch")


def test_e2m1_values_follow_the_format_definition():
    # 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent 0 subnormal
    want = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert [O.e2m1_value(c) for c in range(8)] == want
    assert [O.e2m1_value(c | 8) for c in range(8)] == [-v for v in want]
    assert math.copysign(1.0, O.e2m1_value(8)) == -1.0


@pytest.mark.parametrize("y,code", [
    (0.0, 0), (0.2, 0), (0.25, 0), (0.26, 1), (0.5, 1), (0.75, 2), (1.25, 2), (1.26, 3),
    (1.75, 4), (2.5, 4), (2.51, 5), (3.5, 6), (4.9, 6), (5.0, 6), (5.01, 7), (6.0, 7),
    (7.9, 7), (100.0, 7), (-0.0, 8), (-0.3, 9), (-5.0, 14), (-7.0, 15),
])
def test_hand_derived_roundings(y, code):
    # ties go to the even code: 0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0, 1.75 -> 2.0,
    # 2.5 -> 2.0, 3.5 -> 4.0, 5 -> 4.0; beyond 6 saturates
    assert int(O.e2m1_encode(np.array([y], np.float32))[0]) == code


def test_encoding_is_the_brute_force_nearest_code():
    rng = np.random.default_rng(1)
    y = np.concatenate([rng.uniform(-7, 7, 5000), (np.arange(-14, 15) / 4.0)]).astype(np.float32)
    got = O.e2m1_encode(y)
    vals = np.array([O.e2m1_value(c) for c in range(16)])
    for yi, c in zip(y.astype(np.float64), got):
        d = np.abs(vals - np.clip(yi, -6, 6))
        best = np.flatnonzero(d == d.min())
        best = [b for b in best if np.signbit(vals[b]) == np.signbit(yi) or vals[b] != 0] or list(best)
        if len(best) > 1:                       # a tie between two magnitudes: even code
            best = [b for b in best if b % 2 == 0]
        assert vals[c] == vals[best[0]], (yi, c, best)


@pytest.mark.parametrize("amax,s", [(6.0, 0), (4.0, 0), (7.9, 0), (8.0, 1), (1.0, -2),
                                     (0.75, -3), (65504.0, 13), (2.0 ** -24, -26), (0.0, -127)])
def test_block_scale_follows_the_ocp_rule(amax, s):
    # s = floor(log2 amax) - 2, so amax / 2^s lies in [4, 8)
    block = np.zeros(32, np.float16)
    block[7] = -amax
    block[3] = amax / 3
    assert O.block_exponent(block) == s


def test_largest_magnitude_codes_to_four_or_six():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((50, 128)) * np.exp(rng.uniform(-8, 8, (50, 1)))).astype(np.float16)
    codes, scales = O.quantize_mx(x)
    blocks = x.reshape(50, 4, 32).astype(np.float64)
    c = codes.reshape(50, 4, 32)
    top = np.argmax(np.abs(blocks), axis=2)
    mags = np.take_along_axis(c, top[..., None], axis=2)[..., 0] & 7
    assert set(np.unique(mags)) <= {6, 7}
    assert np.all(scales == np.array([[O.block_exponent(b) + 127 for b in row] for row in blocks.astype(np.float16)]))


def test_values_on_the_grid_round_trip_exactly():
    rng = np.random.default_rng(3)
    mags = rng.integers(0, 8, (10, 128))
    signs = rng.integers(0, 2, (10, 128)) * 8
    s = rng.integers(-20, 10, (10, 4))
    x = np.array([[O.e2m1_value(m | g) for m, g in zip(rm, rg)] for rm, rg in zip(mags, signs)])
    x = (x.reshape(10, 4, 32) * np.exp2(s)[..., None]).reshape(10, 128)
    x[:, ::32] = 6.0 * np.exp2(s)                # each block's largest value fixes its scale
    codes, scales = O.quantize_mx(x.astype(np.float16))
    assert np.array_equal(O.dequantize_mx(codes, scales), x)


def test_quantization_error_is_within_half_a_step():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((40, 128)) * 3).astype(np.float16)
    codes, scales = O.quantize_mx(x)
    xr = O.dequantize_mx(codes, scales).reshape(40, 4, 32)
    X = np.exp2(scales.astype(np.float64) - 127)[..., None]
    err = np.abs(xr - x.reshape(40, 4, 32).astype(np.float64)) / X
    # grid spacing: 0.5 below 2, 1 in [2, 4), 2 in [4, 6]; beyond 6 saturation
    a = np.abs(x.reshape(40, 4, 32).astype(np.float64)) / X
    half = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0))
    assert np.all((err <= half + 1e-12) | (a > 6))


def test_layout_positions():
    codes = np.arange(64, dtype=np.uint8).reshape(1, 64) % 16
    packed = O.pack_nibbles(codes)
    assert packed[0, 0] == (0 | (1 << 4)) and packed[0, 5] == (10 | (11 << 4))
    assert np.array_equal(O.unpack_nibbles(packed), codes)
    T, d = 64, 128
    c = (np.arange(T * d).reshape(T, d) % 16).astype(np.uint8)
    runs = O.pack_mx_value_runs(c)                          # [2, 128, 16]
    for run in range(2):
        for ch in (0, 77):
            for p in range(32):
                t = run * 32 + O.RUN_ORDER[p]
                nib = (runs[run, ch, p // 2] >> (4 * (p % 2))) & 15
                assert nib == c[t, ch]
    sc = (np.arange(T * 4).reshape(T, 4) % 251).astype(np.uint8)
    ps = O.pack_value_scales(sc)                            # [2, 4, 32]
    assert ps[1, 3, 5] == sc[32 + O.RUN_ORDER[5], 3]


def test_appends_equal_prefill():
    rng = np.random.default_rng(5)
    K = (rng.standard_normal((2, 2, 40, 128)) * 2).astype(np.float16)
    V = (rng.standard_normal((2, 2, 40, 128)) * 2).astype(np.float16)
    a = O.MXFP4Cache(2, 2, 128, 64)
    a.prefill(K, V)
    b = O.MXFP4Cache(2, 2, 128, 64)
    b.prefill(K[:, :, :7], V[:, :, :7])
    for t in range(7, 40):
        b.append(K[:, :, t], V[:, :, t])
    for n in ("k", "v", "ks", "vs"):
        assert np.array_equal(getattr(a, n), getattr(b, n))


def test_attention_on_the_grid_is_plain_sdpa():
    rng = np.random.default_rng(6)
    B, H, g, T, d = 1, 2, 4, 70, 128
    grid = np.array([O.e2m1_value(c) for c in range(16)])
    K = grid[rng.integers(0, 16, (B, H, T, d))]
    V = grid[rng.integers(0, 16, (B, H, T, d))] / 2
    K[..., ::32] = 6.0                           # block scales 1 (Keys) and 1/2 (Values)
    V[..., ::32] = 3.0
    c = O.MXFP4Cache(B, H, d, 96)
    c.prefill(K.astype(np.float16), V.astype(np.float16))
    Kd, Vd = c.dequantized()
    assert np.array_equal(Kd, K) and np.array_equal(Vd, V)
    q = rng.standard_normal((B, H * g, d)).astype(np.float16)
    got = c.attend(q, 0.1)
    for j in range(H * g):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[0, j:j + 1].astype(np.float64))[None],
            torch.from_numpy(K[0, j // g])[None], torch.from_numpy(V[0, j // g])[None],
            scale=float(np.float32(0.1)))
        assert np.allclose(got[0, j], ref[0, 0].numpy(), rtol=1e-6, atol=1e-6)
