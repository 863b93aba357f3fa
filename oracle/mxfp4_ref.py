"""CPU oracle for the MXFP4 KV-cache codec and the decode attention that reads it.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or runs this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code with the HIP path.

What the pages fix:
  [LESTY] "KV Cache Quantization (KIVI & FP4)", §4 "Hardware Micro-Scaling": FP4
          micro-scaling (MXFP4) stores four-bit E2M1 numbers (1 sign, 2 exponent,
          1 mantissa bit) in small blocks that share one 8-bit scale, and the matrix
          hardware computes on the four-bit values directly.  The page speaks of
          blocks of 16; the Open Compute Project MX format it names uses blocks of 32
          with a power-of-two (E8M0) scale.

Readings of what the pages leave open (also listed in the design notes):
  R17  The format is OCP MXFP4: blocks of 32 elements share an E8M0 scale X = 2^s
       (code s + 127, s in [-127, 127]); elements are E2M1 (bias 1; magnitudes 0,
       0.5, 1, 1.5, 2, 3, 4, 6).  The scale of a block follows the OCP conversion:
       s = floor(log2(max |x|)) - 2 (2 being E2M1's largest exponent), clamped to
       [-127, 127]; a block of zeros gets s = -127.  Each element is the E2M1 value
       nearest to x / X (exact: X is a power of two), ties to the even code,
       saturating at 6, sign kept.  Decoding: value(code) * X.
  R18  Blocks run along the channels of one token, for Keys and Values alike: a
       token's 128 channels form 4 blocks, so every token is coded on its own when
       it arrives (no window) — the way a decoder writes its cache.
  R19  Layout (a choice of this implementation, part of the bit-exact contract), per
       (sequence, KV head): Key codes [T][d/2] bytes, channel 2i in the low nibble of
       byte i and 2i+1 in the high nibble; Key scales [T][d/32].  Value codes in runs
       of 32 tokens [T/32][d][16] bytes, position p of a channel's run (p = 2i low
       nibble, 2i+1 high nibble of byte i) holding token RUN_ORDER[p] of the run
       (the FP8 codec's order 0-3, 16-19, 4-7, 20-23, ...); Value scales
       [T/32][d/32][32], position p holding token RUN_ORDER[p].  Codes past T in a
       run are 0.
  R20  Attention over the MXFP4 cache: as the KIVI oracle's (reading R7), over the
       decoded Keys and Values, accumulated in float64.
"""
from __future__ import annotations

import numpy as np

from .fp8_ref import RUN_ORDER

F32 = np.float32
BLOCK = 32
V_RUN = 32
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])   # magnitude of codes 0..7
EMAX_ELEM = 2                                               # 6 = 1.5 * 2^2


def e2m1_value(code: int) -> float:
    """Value of a four-bit E2M1 code from the format definition (reading R17): bit 3
    sign, bits 2..1 exponent (bias 1), bit 0 mantissa; exponent 0 is subnormal."""
    code = int(code)
    sign = -1.0 if code & 8 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        return sign * m * 0.5
    return sign * (1.0 + m / 2.0) * 2.0 ** (e - 1)


def e2m1_encode(y: np.ndarray) -> np.ndarray:
    """Nearest E2M1 code of each float32 y, ties to the even code, saturating at 6,
    sign kept (reading R17).  Written as a search of the magnitude table."""
    y = np.asarray(y, F32)
    a = np.abs(y.astype(np.float64)).ravel()
    i = np.clip(np.searchsorted(E2M1, a, side="right") - 1, 0, 7)     # E2M1[i] <= a
    j = np.minimum(i + 1, 7)
    below, above = a - E2M1[i], E2M1[j] - a
    pick_hi = (above < below) | ((above == below) & (j % 2 == 0) & (j != i))
    code = np.where(pick_hi, j, i)
    code = np.where(a >= 6.0, 7, code)
    neg = np.signbit(y.ravel())
    return (code | np.where(neg, 8, 0)).astype(np.uint8).reshape(y.shape)


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    lut = np.array([e2m1_value(c) for c in range(16)], np.float64)
    return lut[np.asarray(codes, np.uint8)]


def block_exponents(blocks: np.ndarray) -> np.ndarray:
    """s of each block (last axis) of float16 values (reading R17): floor(log2 amax)
    is frexp's exponent minus one (exact)."""
    amax = np.max(np.abs(np.asarray(blocks, np.float64)), axis=-1)
    _, e = np.frexp(amax)
    s = np.clip(e.astype(np.int64) - 1 - EMAX_ELEM, -127, 127)
    return np.where(amax == 0.0, -127, s)


def block_exponent(block: np.ndarray) -> int:
    """s of one block of float16 values (reading R17)."""
    return int(block_exponents(np.asarray(block)[None])[0])


def quantize_mx(x: np.ndarray):
    """x float16 [..., n] with n a multiple of 32 -> (codes uint8 [..., n], scale codes
    uint8 [..., n/32]) (reading R17)."""
    x = np.asarray(x, np.float16)
    *lead, n = x.shape
    blocks = x.reshape(*lead, n // BLOCK, BLOCK)
    s = block_exponents(blocks)
    y = blocks.astype(F32) / np.exp2(s.astype(np.float64))[..., None].astype(F32)
    codes = e2m1_encode(y).reshape(*lead, n)
    return codes, (s + 127).astype(np.uint8)


def dequantize_mx(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 value(code) * 2^(scale - 127), blockwise."""
    *lead, n = codes.shape
    v = e2m1_decode(codes).reshape(*lead, n // BLOCK, BLOCK)
    v = v * np.exp2(np.asarray(scales, np.float64) - 127)[..., None]
    return v.reshape(*lead, n)


# ---- storage layout (reading R19) ---------------------------------------------------

def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[..., 2m] four-bit codes -> [..., m] bytes, element 2i in the low nibble."""
    c = np.asarray(codes, np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, np.uint8)
    out = np.empty((*p.shape[:-1], 2 * p.shape[-1]), np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def pack_value_runs(codes: np.ndarray) -> np.ndarray:
    """[..., T, d] Value codes (T a multiple of 32) -> [..., T/32, d, 16] bytes."""
    *lead, T, d = codes.shape
    runs = np.swapaxes(codes.reshape(*lead, T // V_RUN, V_RUN, d), -1, -2)   # [.., d, 32]
    return pack_nibbles(runs[..., RUN_ORDER])


def pack_value_scales(scales: np.ndarray) -> np.ndarray:
    """[..., T, d/32] Value scale codes -> [..., T/32, d/32, 32]."""
    *lead, T, nb = scales.shape
    runs = np.swapaxes(scales.reshape(*lead, T // V_RUN, V_RUN, nb), -1, -2)
    return np.ascontiguousarray(runs[..., RUN_ORDER])


class MXFP4Cache:
    """MXFP4 K/V of one layer: element codes and block scale codes per token,
    [B][H][T][d] and [B][H][T][d/32] (the packing of reading R19 is applied by the
    pack_* functions when comparing with a device cache)."""

    def __init__(self, batch, kv_heads, head_dim, max_tokens):
        self.B, self.H, self.d, self.Tmax = batch, kv_heads, head_dim, max_tokens
        self.k = np.zeros((batch, kv_heads, max_tokens, head_dim), np.uint8)
        self.v = np.zeros_like(self.k)
        self.ks = np.zeros((batch, kv_heads, max_tokens, head_dim // BLOCK), np.uint8)
        self.vs = np.zeros_like(self.ks)
        self.T = 0

    def _store(self, K, V, t0):
        n = K.shape[2]
        self.k[:, :, t0:t0 + n], self.ks[:, :, t0:t0 + n] = quantize_mx(K)
        self.v[:, :, t0:t0 + n], self.vs[:, :, t0:t0 + n] = quantize_mx(V)

    def prefill(self, K: np.ndarray, V: np.ndarray):
        """K, V float16 [B][H][T][d]: every token is coded on its own (reading R18)."""
        self._store(K, V, 0)
        self.T = K.shape[2]

    def append(self, k_new: np.ndarray, v_new: np.ndarray):
        """k_new, v_new float16 [B][H][d]."""
        self._store(k_new[:, :, None, :], v_new[:, :, None, :], self.T)
        self.T += 1

    def dequantized(self):
        T = self.T
        K = dequantize_mx(self.k[:, :, :T], self.ks[:, :, :T])
        V = dequantize_mx(self.v[:, :, :T], self.vs[:, :, :T])
        return K, V

    def attend(self, q: np.ndarray, sm_scale: float) -> np.ndarray:
        """q float16 [B][H_q][d] -> float32 [B][H_q][d]; query head j reads KV head
        j // (H_q / H) (reading R6), softmax attention in float64 (reading R20)."""
        from .kivi_ref import gqa_attention_fp64
        K, V = self.dequantized()
        return gqa_attention_fp64(q, K, V, sm_scale)
