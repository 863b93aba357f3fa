"""CPU oracle for the FP8 KV-cache codec and the decode attention that reads it.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or runs this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code with the HIP path.

What the pages fix:
  [FORT]  "09 — KV Cache Quantization", "The lazy default: FP8 KV": the cache is
          stored as FP8 in the E4M3 or the E5M2 format, halving float16 storage.
  [INFRA] "4.4 KV Cache quantization" §4.1 (the two formats: E4M3 more precision,
          E5M2 more range), §4.2 (real values need a scale to land in FP8's range;
          one scale per tensor or one per attention head; 1.0 when uncalibrated),
          §4.5 (the stored precision is not the compute precision: a backend may
          widen the codes before attending).

Readings of what the pages leave open (also listed in the design notes):
  R11  The formats are the OCP 8-bit floating point formats: E4M3 with exponent
       bias 7, no infinities, the all-ones pattern (0x7F / 0xFF) NaN, largest finite
       value 448; E5M2 with exponent bias 15 and IEEE-style infinities (0x7C) and
       NaNs, largest finite value 57344.  Both have subnormals.
  R12  Encoding: code = the FP8 value nearest to float32(x) / s (IEEE float32
       division, s the float32 scale of the (KV head, K or V)), ties to the even
       code, saturating: magnitudes beyond the largest finite value give it.  The
       sign is kept (-0.0 gives 0x80).  Decoding: float32(value(code)) * s.  Scales
       are per KV head; a per-tensor scale is the same value for every head.
  R13  Attention over the FP8 cache: as the KIVI oracle's (reading R7: the new token
       is stored first, then the query attends over all T tokens), over the decoded
       Keys and Values, accumulated in float64.
  R14  Layout (a choice of this implementation, part of the bit-exact contract):
       Key codes ``[T][d]`` per (sequence, KV head); Value codes in runs of 32 tokens
       ``[T/32][d][32]``, the 32 bytes of a channel holding the run's tokens in the
       order 0-3, 16-19, 4-7, 20-23, 8-11, 24-27, 12-15, 28-31.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
V_RUN = 32
# position p of a Value run holds token RUN_ORDER[p] of the run (reading R14)
RUN_ORDER = np.array([4 * (p // 8) + (p % 4) + 16 * ((p % 8) // 4) for p in range(V_RUN)])

FORMATS = {
    # name: (exponent bits, mantissa bits, bias, largest finite value)
    "e4m3": (4, 3, 7, 448.0),
    "e5m2": (5, 2, 15, 57344.0),
}


def fp8_value(code: int, fmt: str) -> float:
    """The real value of an FP8 code, from the format definition (reading R11)."""
    E, M, bias, _ = FORMATS[fmt]
    code = int(code)                            # no uint8 wrap-around below
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> M) & ((1 << E) - 1)
    m = code & ((1 << M) - 1)
    if fmt == "e4m3" and e == 15 and m == 7:
        return float("nan")
    if fmt == "e5m2" and e == 31:
        return sign * float("inf") if m == 0 else float("nan")
    if e == 0:                                   # subnormal: m * 2^(1 - bias - M)
        return sign * m * 2.0 ** (1 - bias - M)
    return sign * (1.0 + m / 2.0 ** M) * 2.0 ** (e - bias)


def finite_table(fmt: str):
    """Non-negative finite codes of the format and their values, in increasing order."""
    codes = [c for c in range(0x80) if np.isfinite(fp8_value(c, fmt))]
    vals = np.array([fp8_value(c, fmt) for c in codes], np.float64)
    assert np.all(np.diff(vals) > 0)
    return np.array(codes, np.uint8), vals


def fp8_encode(y: np.ndarray, fmt: str) -> np.ndarray:
    """Nearest FP8 code of each float32 y, ties to the even code, saturating
    (reading R12).  Written as a search of the table of finite values."""
    y = np.asarray(y, F32)
    codes, vals = finite_table(fmt)
    a = np.abs(y.astype(np.float64)).ravel()
    if not np.all(np.isfinite(a)):
        raise ValueError("inputs must be finite")
    i = np.clip(np.searchsorted(vals, a, side="right") - 1, 0, len(vals) - 1)   # vals[i] <= a
    j = np.minimum(i + 1, len(vals) - 1)
    lo, hi = vals[i], vals[j]
    below = a - lo
    above = hi - a
    pick_hi = (above < below) | ((above == below) & (codes[j] % 2 == 0) & (j != i))
    out = np.where(pick_hi, codes[j], codes[i]).astype(np.uint8)
    out = np.where(a >= vals[-1], codes[-1], out)           # saturate
    neg = np.signbit(y.ravel())
    return (out | np.where(neg, 0x80, 0).astype(np.uint8)).reshape(y.shape)


def fp8_decode(codes: np.ndarray, fmt: str) -> np.ndarray:
    """float32 value of each code."""
    lut = np.array([fp8_value(c, fmt) for c in range(256)], np.float64).astype(F32)
    return lut[np.asarray(codes, np.uint8)]


def quantize_fp8(x: np.ndarray, scale, fmt: str) -> np.ndarray:
    """codes = encode(float32(x) / s), float32 division (reading R12)."""
    return fp8_encode(np.asarray(x, np.float32) / F32(scale), fmt)


def dequantize_fp8(codes: np.ndarray, scale, fmt: str) -> np.ndarray:
    """float32(value(code)) * s."""
    return fp8_decode(codes, fmt) * F32(scale)


def pack_value_runs(codes: np.ndarray) -> np.ndarray:
    """[..., T, d] Value codes (T a multiple of 32) -> [..., T/32, d, 32] (reading R14)."""
    *lead, T, d = codes.shape
    runs = codes.reshape(*lead, T // V_RUN, V_RUN, d)
    runs = np.swapaxes(runs, -1, -2)                       # [..., T/32, d, 32 tokens]
    return np.ascontiguousarray(runs[..., RUN_ORDER])


def unpack_value_runs(packed: np.ndarray) -> np.ndarray:
    *lead, nrun, d, _ = packed.shape
    runs = np.empty_like(packed)
    runs[..., RUN_ORDER] = packed
    return np.ascontiguousarray(np.swapaxes(runs, -1, -2).reshape(*lead, nrun * V_RUN, d))


class FP8Cache:
    """FP8 K/V of one layer: codes [B][H][T][d] and per-KV-head float32 scales."""

    def __init__(self, batch, kv_heads, head_dim, fmt, max_tokens, k_scale, v_scale):
        self.B, self.H, self.d, self.fmt, self.Tmax = batch, kv_heads, head_dim, fmt, max_tokens
        # one scale per KV head; a single value is a per-tensor scale (every head)
        self.k_scale = np.broadcast_to(np.asarray(k_scale, F32), (kv_heads,)).copy()
        self.v_scale = np.broadcast_to(np.asarray(v_scale, F32), (kv_heads,)).copy()
        self.k = np.zeros((batch, kv_heads, max_tokens, head_dim), np.uint8)
        self.v = np.zeros((batch, kv_heads, max_tokens, head_dim), np.uint8)
        self.T = 0

    def _store(self, K: np.ndarray, V: np.ndarray, t0: int):
        n = K.shape[2]
        for h in range(self.H):
            self.k[:, h, t0:t0 + n] = quantize_fp8(K[:, h], self.k_scale[h], self.fmt)
            self.v[:, h, t0:t0 + n] = quantize_fp8(V[:, h], self.v_scale[h], self.fmt)

    def prefill(self, K: np.ndarray, V: np.ndarray):
        """K, V float16 [B][H][T][d]: every token is coded on its own."""
        self._store(K, V, 0)
        self.T = K.shape[2]

    def append(self, k_new: np.ndarray, v_new: np.ndarray):
        """k_new, v_new float16 [B][H][d]."""
        self._store(k_new[:, :, None, :], v_new[:, :, None, :], self.T)
        self.T += 1

    def dequantized(self):
        T = self.T
        K = np.empty((self.B, self.H, T, self.d), F32)
        V = np.empty_like(K)
        for h in range(self.H):
            K[:, h] = dequantize_fp8(self.k[:, h, :T], self.k_scale[h], self.fmt)
            V[:, h] = dequantize_fp8(self.v[:, h, :T], self.v_scale[h], self.fmt)
        return K, V

    def attend(self, q: np.ndarray, sm_scale: float) -> np.ndarray:
        """q float16 [B][H_q][d] -> float32 [B][H_q][d]; query head j reads KV head
        j // (H_q / H) (reading R6), softmax attention in float64 (reading R13)."""
        from .kivi_ref import gqa_attention_fp64
        K, V = self.dequantized()
        return gqa_attention_fp64(q, K, V, sm_scale)
