"""Pins of the FP8 oracle (oracle/fp8_ref.py) against what the format definitions and
independent routines fix: closed-form code values, torch's own float8 conversion for
in-range values (round to nearest, ties to even), exhaustive round trips, saturation,
the Value-run layout, and attention that reduces to plain SDPA when the data is on
the FP8 grid."""
import math

import numpy as np
import pytest

import oracle as O

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("fmt,code,value", [
    ("e4m3", 0x00, 0.0), ("e4m3", 0x01, 2.0 ** -9), ("e4m3", 0x07, 7 * 2.0 ** -9),
    ("e4m3", 0x08, 2.0 ** -6), ("e4m3", 0x38, 1.0), ("e4m3", 0x3F, 1.875), ("e4m3", 0x40, 2.0),
    ("e4m3", 0x7E, 448.0), ("e4m3", 0xFE, -448.0), ("e4m3", 0xB8, -1.0),
    ("e5m2", 0x01, 2.0 ** -16), ("e5m2", 0x03, 3 * 2.0 ** -16), ("e5m2", 0x04, 2.0 ** -14),
    ("e5m2", 0x3C, 1.0), ("e5m2", 0x3D, 1.25), ("e5m2", 0x7B, 57344.0), ("e5m2", 0xFB, -57344.0),
])
def test_code_values_follow_the_format_definitions(fmt, code, value):
    assert O.fp8_value(code, fmt) == value


def test_special_codes_and_counts():
    assert math.isnan(O.fp8_value(0x7F, "e4m3")) and math.isnan(O.fp8_value(0xFF, "e4m3"))
    assert O.fp8_value(0x7C, "e5m2") == math.inf and O.fp8_value(0xFC, "e5m2") == -math.inf
    assert all(math.isnan(O.fp8_value(c, "e5m2")) for c in (0x7D, 0x7E, 0x7F))
    assert math.copysign(1.0, O.fp8_value(0x80, "e4m3")) == -1.0
    # non-negative finite codes: e4m3 0x00..0x7E, e5m2 0x00..0x7B
    assert len(O.finite_table("e4m3")[0]) == 127 and len(O.finite_table("e5m2")[0]) == 124


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_every_finite_code_round_trips(fmt):
    codes, _ = O.finite_table(fmt)
    for c in list(codes) + [int(x) | 0x80 for x in codes]:
        y = np.array([O.fp8_value(c, fmt)], np.float32)
        assert int(O.fp8_encode(y, fmt)[0]) == c


@pytest.mark.parametrize("fmt,tdt", [("e4m3", "float8_e4m3fn"), ("e5m2", "float8_e5m2")])
def test_encoding_matches_torch_float8_in_range(fmt, tdt):
    # torch converts with round-to-nearest-even but does not saturate, so compare where
    # rounding cannot overflow: below the largest value plus half its spacing
    dt = getattr(torch, tdt)
    _, vals = O.finite_table(fmt)
    top = vals[-1] + (vals[-1] - vals[-2]) / 2
    rng = np.random.default_rng(4)
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)          # every tie
    near = np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0))
    wide = np.exp(rng.uniform(np.log(1e-7), np.log(top), 20000)).astype(np.float32)
    y = np.concatenate([mids, *near, wide, vals.astype(np.float32)])
    y = y[y < top]
    y = np.concatenate([y, -y])
    ref = torch.from_numpy(y).to(dt).view(torch.uint8).numpy()
    got = O.fp8_encode(y, fmt)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, (y[bad[:5]], got[bad[:5]], ref[bad[:5]])


def test_ties_go_to_the_even_code_and_large_values_saturate():
    e = lambda v, f="e4m3": int(O.fp8_encode(np.array([v], np.float32), f)[0])
    assert e(1.0625) == 0x38 and e(1.1875) == 0x3A           # 1 | 1.125 | 1.25
    assert e(0.5 * 2 ** -9) == 0x00 and e(1.5 * 2 ** -9) == 0x02
    assert e(460.0) == 0x7E and e(470.0) == 0x7E and e(1e30) == 0x7E and e(-1e30) == 0xFE
    assert e(61440.0, "e5m2") == 0x7B and e(-1e9, "e5m2") == 0xFB
    assert e(-0.0) == 0x80 and e(0.0) == 0x00


def test_quantize_divides_by_the_scale_in_float32():
    x = np.array([3.0, -7.5, 0.05, 150.0], np.float16)          # x / s normal and in range
    s = np.float32(0.37)
    y = x.astype(np.float32) / s
    assert np.array_equal(O.quantize_fp8(x, s, "e4m3"), O.fp8_encode(y, "e4m3"))
    back = O.dequantize_fp8(O.quantize_fp8(x, s, "e4m3"), s, "e4m3")
    # e4m3 keeps 3 mantissa bits: |x - x_hat| <= 2^-4 |x| away from subnormals
    assert np.all(np.abs(back - x.astype(np.float32)) <= 2.0 ** -4 * np.abs(x.astype(np.float32)) + 1e-6)
    # beyond the range the code saturates: 300 / 0.37 > 448
    assert O.quantize_fp8(np.array([300.0], np.float16), s, "e4m3")[0] == 0x7E


def test_value_run_layout():
    assert sorted(O.RUN_ORDER.tolist()) == list(range(32))
    assert O.RUN_ORDER[:8].tolist() == [0, 1, 2, 3, 16, 17, 18, 19]
    assert O.RUN_ORDER[8:16].tolist() == [4, 5, 6, 7, 20, 21, 22, 23]
    codes = np.arange(64 * 4, dtype=np.int64).reshape(64, 4) % 251
    p = O.pack_value_runs(codes.astype(np.uint8))
    assert p.shape == (2, 4, 32)
    assert p[1, 2, 4] == codes[32 + 16, 2]                    # run 1, channel 2, token 16
    assert np.array_equal(O.unpack_value_runs(p), codes.astype(np.uint8))


def test_attention_on_grid_values_is_plain_sdpa():
    # every value exactly representable after division by its head's scale (a power of
    # two): the FP8 cache decodes to the input itself, so attention is SDPA (float64)
    rng = np.random.default_rng(8)
    B, H, g, T, d = 1, 2, 3, 40, 128
    _, vals = O.finite_table("e4m3")
    pick = lambda *shape: (vals[rng.integers(0, 80, shape)] * rng.choice([-1, 1], shape))
    ks, vs = np.array([0.5, 2.0], np.float32), np.array([4.0, 0.25], np.float32)
    K = (pick(B, H, T, d) * ks[None, :, None, None]).astype(np.float16)
    V = (pick(B, H, T, d) * vs[None, :, None, None]).astype(np.float16)
    c = O.FP8Cache(B, H, d, "e4m3", 64, ks, vs)
    c.prefill(K, V)
    q = rng.standard_normal((B, H * g, d)).astype(np.float16)
    got = c.attend(q, 0.1)
    for j in range(H * g):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[:, j:j + 1].astype(np.float64))[None],
            torch.from_numpy(K[:, j // g].astype(np.float64))[None],
            torch.from_numpy(V[:, j // g].astype(np.float64))[None], scale=float(np.float32(0.1)))
        assert np.allclose(got[:, j], ref[0, :, 0].numpy(), rtol=1e-6, atol=1e-6)


def test_append_equals_prefill():
    rng = np.random.default_rng(9)
    B, H, T, d = 2, 2, 37, 128
    K = (rng.standard_normal((B, H, T, d)) * 30).astype(np.float16)
    V = (rng.standard_normal((B, H, T, d)) * 30).astype(np.float16)
    a = O.FP8Cache(B, H, d, "e5m2", 64, [1.0, 0.5], [2.0, 1.0])
    b = O.FP8Cache(B, H, d, "e5m2", 64, [1.0, 0.5], [2.0, 1.0])
    a.prefill(K, V)
    b.prefill(K[:, :, :20], V[:, :, :20])
    for t in range(20, T):
        b.append(K[:, :, t], V[:, :, t])
    assert np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v) and a.T == b.T
