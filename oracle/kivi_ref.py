"""CPU oracle for KIVI-style KV-cache quantization and decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or runs this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code with the HIP path (no kernels, headers,
tables or helpers); the two meet only in the seeded inputs of ``workloads``.

Everything here is written to be checked by eye against the pages:

  [LESTY]   "KV Cache Quantization (KIVI & FP4): How 2-Bit Key-Value Compression
            Scales LLM Contexts to 1 Million Tokens" (lesty.tech)
  [FORT]    "09 — KV Cache Quantization" (project-fortress)
  [ZSM]     "KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV Cache"
            (zeroshotmind)
  [INFRA]   "4.4 KV Cache quantization" (infra-guide)
  [ZYEKH]   "KV Cache INT4 Quantization for 1M+ Token Context Windows" (zyekh)

Precision: the quantizer runs in float32 with IEEE semantics (no fused
multiply-add, correctly rounded division, round-half-to-even, float32->float16 by
round-to-nearest-even); attention accumulates in float64 and returns float32.
Every numpy scalar below is an explicit ``np.float32`` so that numpy's type
promotion never silently widens a float32 step to float64.

Readings of passages the pages leave open (each is also listed in the design notes):
  R1  zero := the group minimum stored as float16 (exact); codes are
      ``rint((x - min) / scale)`` with the *stored* float16 scale, clamped to
      [0, 2^b - 1].  [ZYEKH] §2 prints an integer zero-point form; that form cannot
      represent near-constant groups in float16, so the minimum itself is the zero.
  R2  scale == 0 (constant group, or a range that underflows float16) gives all
      codes 0 and dequantizes every element to the minimum.
  R3  -0.0 inputs are canonicalized to +0.0 before min/max.
  R4  Value groups: G_v consecutive channels of one token, starting at channel 0.
      Key groups: G consecutive tokens of one channel, starting at token 0.
  R5  Residual window: one window shared by K and V holding r(T) = ((T-1) mod R)+1
      tokens (0 when T == 0); it is flushed whole, when it is full and a new token
      arrives.  Prefill of T tokens produces the same state as T appends.
  R6  GQA: query head j reads KV head j // (H_q / H_kv).
  R7  Decode step order: append the new token (flushing first if the window is
      full), then attend over all T tokens including the new one; no mask.
  R8  Packed layout (the pages fix four 2-bit or two 4-bit codes per byte, but
      neither the bit order nor the pack axis): a packed run is cut into
      little-endian 32-bit words of n = 32/b codes, and code e of a word sits in
      byte e mod 4 at bits [b*(e div 4), b*(e div 4) + b) ("word-interleaved"
      order: byte k of a word holds codes k, k+4, k+8, ...).  Keys: per token,
      along channels ``[T][d*b/8]``.  Values: per channel, along runs of 16 tokens
      ``[T/16][d][16*b/8]``.  Each product of decode attention then reduces along
      the packed axis (Q.K^T over channels, P.V over tokens), and a shift by b*k
      and a byte mask extract codes 4k .. 4k+3 of a word in their natural order.
  R15 Sink tokens ([FORT] "Anti-patterns": the first few tokens absorb large
      attention scores and must not be quantized; preserve the first N): with S sink
      tokens, tokens [0, S) of a sequence stay in float16 for its lifetime and every
      rule above (groups, window, flushes) applies to tokens S, S+1, ... counted
      from S.  S = 0 is the plain method.
  R16 Group-wise aging of the window ([ZSM] "The streaming complication": as the
      window fills, a completed group of keys is quantized once and frozen, and the
      newest tokens stay in float16 until they age out).  Variant of R5, selected
      per cache: the window holds at most R tokens; a token that arrives at a full
      window first sends only the oldest G window tokens (one Key group; their
      Values token by token) into the history, and the newest R - G stay.  Hence
      r(T) = T for T <= R and R - G + ((T - R - 1) mod G) + 1 after, so the window
      always keeps at least the R - G + 1 most recent tokens.  G = R is R5.
  R21 Per-token Value window ([INFRA] §3.2: a Value needs no group to fill, and its
      residual keeps only the most recent tokens, each arrival pushing the oldest
      one out after quantizing it, like a sliding window).  Variant selected per
      cache (``v_window="token"``; the default "flush" moves Values with the Keys as
      in R5/R16): the Value window holds exactly the min(T_k, R) most recent tokens
      after the sink, and a token that arrives at a full Value window first
      quantizes the oldest one (on its own, G_v-channel groups) into history
      position T_k - R.  Keys keep their rule.  Tokens in [T_k - R, T_k - r) then
      have quantized Keys and float16 Values.
"""
from __future__ import annotations

import math

import numpy as np

F32 = np.float32
F16 = np.float16
V_RUN = 16  # tokens per packed Value run (reading R8)


# --------------------------------------------------------------------------------------
# Memory accounting
# --------------------------------------------------------------------------------------

def kv_cache_bytes(layers: int, batch: int, tokens: int, kv_heads: int, head_dim: int,
                   bytes_per_elem: float) -> float:
    """M_KV = 2 * L * B * T * H_kv * d * b  (the leading 2 counts K and V).

    [INFRA] §1 "First estimate how much cache you can save"; [LESTY] §1;
    [FORT] "The number that motivates everything".
    """
    return 2 * layers * batch * tokens * kv_heads * head_dim * bytes_per_elem


def residual_len(T: int, R: int) -> int:
    """Tokens held in the float16 residual window after T tokens (reading R5)."""
    return 0 if T == 0 else (T - 1) % R + 1


def quantized_len(T: int, R: int) -> int:
    return T - residual_len(T, R)


def residual_len_grouped(T: int, R: int, G: int) -> int:
    """Window tokens after T tokens when the window ages one Key group at a time
    (reading R16)."""
    return T if T <= R else R - G + (T - R - 1) % G + 1


AGING = ("window", "group")
V_WINDOW = ("flush", "token")


def kivi_cache_bytes(layers: int, batch: int, tokens: int, kv_heads: int, head_dim: int,
                     bits: int, group_k: int, group_v: int, residual: int) -> dict:
    """Bytes held by the quantized cache at T tokens, metadata and residual included.

    [INFRA] §1 notes that the b-bit count alone is a lower bound because it leaves out
    per-group scale/zero and the high-precision residual; those are counted here.
    """
    Tq = quantized_len(tokens, residual)
    r = tokens - Tq
    unit = layers * batch * kv_heads
    codes = 2 * unit * Tq * head_dim * bits // 8
    k_meta = unit * (Tq // group_k) * head_dim * 2 * 2       # fp16 scale + zero
    v_meta = unit * Tq * (head_dim // group_v) * 2 * 2
    resid = 2 * unit * r * head_dim * 2
    return {"codes": codes, "k_meta": k_meta, "v_meta": v_meta, "residual": resid,
            "total": codes + k_meta + v_meta + resid}


# --------------------------------------------------------------------------------------
# The asymmetric min/max quantizer
# --------------------------------------------------------------------------------------

def quantize_groups(x: np.ndarray, bits: int):
    """Quantize each group (the last axis of ``x``) with its own min/max scale and zero.

    Follows the in-group mapping of [INFRA] §3.1 (min/max asymmetric), the float16
    scale and zero of [FORT] "KIVI — the reference paper", and the step size
    range / (2^b - 1) of [ZYEKH] §2 and [LESTY] §6.5, with readings R1-R3.

    Returns (codes uint8 [..., n], scale float16 [...], zero float16 [...]).
    """
    assert x.dtype == F16
    qmax = F32(2 ** bits - 1)
    xf = x.astype(F32) + F32(0.0)                  # R3: -0.0 -> +0.0
    mn = xf.min(axis=-1, keepdims=True)
    mx = xf.max(axis=-1, keepdims=True)
    rng = (mx - mn).astype(F32)                    # float32, round-to-nearest-even
    s32 = (rng / qmax).astype(F32)                 # IEEE float32 division
    scale = s32.astype(F16)                        # float16 RNE
    zero = mn.astype(F16)                          # exact: mn is a float16 value
    s = scale.astype(F32)
    safe = np.where(s == F32(0.0), F32(1.0), s).astype(F32)
    q = np.rint(((xf - mn).astype(F32) / safe).astype(F32))   # rint: ties to even
    q = np.clip(q, F32(0.0), qmax)
    q = np.where(s == F32(0.0), F32(0.0), q)       # R2
    return q.astype(np.uint8), scale[..., 0], zero[..., 0]


def dequantize(codes: np.ndarray, scale: np.ndarray, zero: np.ndarray) -> np.ndarray:
    """x_hat = float32(code) * scale + zero, in float32 (two roundings)."""
    return (codes.astype(F32) * scale.astype(F32)).astype(F32) + zero.astype(F32)


def quantize_keys(K: np.ndarray, G: int, bits: int):
    """Per-channel Key quantization over groups of G consecutive tokens.

    [INFRA] §3.1 (fix a channel, group consecutive tokens: the vertical cut);
    [LESTY] §3 (each Key channel gets its own scale); [ZSM] "Quantize along the axis
    that hides the outliers".

    K: float16 [..., T, d] with T a multiple of G.
    Returns codes uint8 [..., T, d], scale/zero float16 [..., T/G, d].
    """
    *lead, T, d = K.shape
    assert T % G == 0
    g = K.reshape(*lead, T // G, G, d)
    g = np.swapaxes(g, -1, -2)                     # [..., T/G, d, G]: one group per row
    codes, scale, zero = quantize_groups(np.ascontiguousarray(g), bits)
    codes = np.swapaxes(codes, -1, -2).reshape(*lead, T, d)
    return codes, scale, zero


def dequantize_keys(codes: np.ndarray, scale: np.ndarray, zero: np.ndarray, G: int):
    *lead, T, d = codes.shape
    s = np.repeat(scale, G, axis=-2)
    z = np.repeat(zero, G, axis=-2)
    return dequantize(codes, s, z)


def quantize_values(V: np.ndarray, Gv: int, bits: int):
    """Per-token Value quantization over groups of Gv consecutive channels.

    [INFRA] §3.1 (fix a token, group along channels: the horizontal cut);
    [LESTY] §3 (each token slice gets its own scale); [FORT] "The structural fact
    that makes KV quant work".

    V: float16 [..., T, d] with d a multiple of Gv.
    Returns codes uint8 [..., T, d], scale/zero float16 [..., T, d/Gv].
    """
    *lead, T, d = V.shape
    assert d % Gv == 0
    g = V.reshape(*lead, T, d // Gv, Gv)
    codes, scale, zero = quantize_groups(np.ascontiguousarray(g), bits)
    return codes.reshape(*lead, T, d), scale, zero


def dequantize_values(codes: np.ndarray, scale: np.ndarray, zero: np.ndarray, Gv: int):
    s = np.repeat(scale, Gv, axis=-1)
    z = np.repeat(zero, Gv, axis=-1)
    return dequantize(codes, s, z)


# --------------------------------------------------------------------------------------
# Bit packing (reading R8).  [LESTY] §4: four 2-bit codes per byte; [ZYEKH] §2: two
# 4-bit codes per byte.
# --------------------------------------------------------------------------------------

def pack_words(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack the last axis (reading R8): 32-bit little-endian words of n = 32/b codes,
    code e of a word in byte e % 4 at bit offset b * (e // 4)."""
    n = 32 // bits
    *lead, m = codes.shape
    assert m % n == 0
    c = codes.reshape(*lead, m // n, n).astype(np.uint32)
    words = np.zeros((*lead, m // n), np.uint32)
    for e in range(n):
        words |= (c[..., e] & (2 ** bits - 1)) << (8 * (e % 4) + bits * (e // 4))
    return np.ascontiguousarray(words.astype("<u4")).view(np.uint8).reshape(*lead, m * bits // 8)


def unpack_words(packed: np.ndarray, bits: int) -> np.ndarray:
    n = 32 // bits
    *lead, nb = packed.shape
    assert nb % 4 == 0
    words = np.ascontiguousarray(packed).reshape(*lead, nb // 4, 4).view("<u4")[..., 0]
    words = words.astype(np.uint32)
    parts = [(words >> (8 * (e % 4) + bits * (e // 4))) & (2 ** bits - 1) for e in range(n)]
    return np.stack(parts, axis=-1).reshape(*lead, (nb // 4) * n).astype(np.uint8)


def pack_keys(codes: np.ndarray, bits: int) -> np.ndarray:
    """[..., T, d] codes -> [..., T, d*b/8] bytes (per token, along channels)."""
    return pack_words(codes, bits)


def unpack_keys(packed: np.ndarray, bits: int) -> np.ndarray:
    return unpack_words(packed, bits)


def pack_values(codes: np.ndarray, bits: int) -> np.ndarray:
    """[..., T, d] codes -> [..., T/16, d, 16*b/8] bytes (per channel, along tokens)."""
    *lead, T, d = codes.shape
    assert T % V_RUN == 0
    runs = codes.reshape(*lead, T // V_RUN, V_RUN, d)
    runs = np.swapaxes(runs, -1, -2)               # [..., T/16, d, 16]
    return pack_words(np.ascontiguousarray(runs), bits)


def unpack_values(packed: np.ndarray, bits: int) -> np.ndarray:
    runs = unpack_words(packed, bits)              # [..., T/16, d, 16]
    runs = np.swapaxes(runs, -1, -2)               # [..., T/16, 16, d]
    *lead, nr, _, d = runs.shape
    return np.ascontiguousarray(runs).reshape(*lead, nr * V_RUN, d)


# --------------------------------------------------------------------------------------
# One layer of the quantized cache and its streaming state machine
# --------------------------------------------------------------------------------------

class LayerCache:
    """Host model of one layer's quantized KV cache for B sequences x H_kv heads.

    Storage mirrors the device layout (reading R8):
      k_codes  uint8   [B, H, T_max, d*b/8]
      k_scale  float16 [B, H, T_max/G, d]      k_zero likewise
      v_codes  uint8   [B, H, T_max/16, d, 16*b/8]
      v_scale  float16 [B, H, T_max, d/G_v]    v_zero likewise
      k_resid  float16 [B, H, R, d]            v_resid likewise

    [ZSM] "The streaming complication": recent keys stay in full precision and only
    complete groups are quantized, once, then frozen.  [INFRA] §3.2: the residual
    joins attention together with the quantized history and moves into it in a
    batch once enough tokens have accumulated.  [LESTY] §3: the most recent tokens
    are held unquantized in FP16.
    """

    def __init__(self, batch, kv_heads, head_dim, bits, group_k, group_v, residual,
                 max_tokens, sink: int = 0, aging: str = "window", v_window: str = "flush"):
        assert bits in (2, 4) and aging in AGING and v_window in V_WINDOW
        assert residual % group_k == 0 and residual % V_RUN == 0
        assert max_tokens % group_k == 0 and max_tokens % V_RUN == 0
        assert head_dim % group_v == 0
        self.B, self.H, self.d = batch, kv_heads, head_dim
        self.bits, self.G, self.Gv, self.R = bits, group_k, group_v, residual
        self.T_max = max_tokens
        B, H, d = batch, kv_heads, head_dim
        self.k_codes = np.zeros((B, H, max_tokens, d * bits // 8), np.uint8)
        self.k_scale = np.zeros((B, H, max_tokens // group_k, d), F16)
        self.k_zero = np.zeros((B, H, max_tokens // group_k, d), F16)
        self.v_codes = np.zeros((B, H, max_tokens // V_RUN, d, V_RUN * bits // 8), np.uint8)
        self.v_scale = np.zeros((B, H, max_tokens, d // group_v), F16)
        self.v_zero = np.zeros((B, H, max_tokens, d // group_v), F16)
        self.k_resid = np.zeros((B, H, residual, d), F16)
        self.v_resid = np.zeros((B, H, residual, d), F16)
        self.S = sink                       # reading R15
        self.aging = aging                  # reading R5 ("window") or R16 ("group")
        self.v_window = v_window            # reading R21 ("token") or with the Keys
        # R21: the unpacked Value codes of the history (a token's codes are written
        # on their own and its 16-token run is packed again)
        self.v_code_vals = np.zeros((B, H, max_tokens, d), np.uint8)
        self.k_sink = np.zeros((B, H, sink, d), F16)
        self.v_sink = np.zeros((B, H, sink, d), F16)
        self.T = 0

    @property
    def Tk(self) -> int:
        """Tokens under the KIVI rules: those after the sink (reading R15)."""
        return max(0, self.T - self.S)

    def window_len(self, Tk: int) -> int:
        """r: window tokens when Tk tokens follow the sink (readings R5 and R16)."""
        if self.aging == "group":
            return residual_len_grouped(Tk, self.R, self.G)
        return residual_len(Tk, self.R)

    @property
    def Tq(self) -> int:
        """Tokens in the quantized Key history (and Value history unless R21)."""
        return self.Tk - self.window_len(self.Tk)

    @property
    def Tqv(self) -> int:
        """Tokens in the quantized Value history."""
        if self.v_window == "token":
            return max(0, self.Tk - self.R)
        return self.Tq

    # -- writes into the quantized store ------------------------------------------------
    def _store(self, K: np.ndarray, V: np.ndarray, t0: int):
        """Quantize tokens K/V [B, H, n, d] (n a multiple of G) into offset t0."""
        self._store_k(K, t0)
        self._store_v(V, t0)

    def _store_k(self, K: np.ndarray, t0: int):
        n = K.shape[2]
        kc, ks, kz = quantize_keys(K, self.G, self.bits)
        self.k_codes[:, :, t0:t0 + n] = pack_keys(kc, self.bits)
        self.k_scale[:, :, t0 // self.G:(t0 + n) // self.G] = ks
        self.k_zero[:, :, t0 // self.G:(t0 + n) // self.G] = kz

    def _store_v(self, V: np.ndarray, t0: int):
        """Quantize Value tokens [B, H, n, d] into history positions t0 .. t0 + n - 1;
        any n (each token is coded on its own), its runs packed again."""
        n = V.shape[2]
        vc, vs, vz = quantize_values(V, self.Gv, self.bits)
        self.v_code_vals[:, :, t0:t0 + n] = vc
        self.v_scale[:, :, t0:t0 + n] = vs
        self.v_zero[:, :, t0:t0 + n] = vz
        r0, r1 = t0 // V_RUN, (t0 + n + V_RUN - 1) // V_RUN
        self.v_codes[:, :, r0:r1] = pack_values(
            self.v_code_vals[:, :, r0 * V_RUN:r1 * V_RUN], self.bits)

    def prefill(self, K: np.ndarray, V: np.ndarray):
        """Quantize a prompt of T tokens at once (T quantized + r residual, reading R5).

        [LESTY] §6: prefill runs in full precision and a streaming pass then stores
        the history in low-bit form.
        """
        assert K.dtype == F16 and V.dtype == F16 and K.shape == V.shape
        T = K.shape[2]
        assert T + 1 <= self.T_max
        ns = min(T, self.S)
        self.k_sink[:, :, :ns] = K[:, :, :ns]
        self.v_sink[:, :, :ns] = V[:, :, :ns]
        K, V = K[:, :, ns:], V[:, :, ns:]
        Tk = T - ns
        r = self.window_len(Tk)
        Tq = Tk - r
        if Tq:
            self._store_k(K[:, :, :Tq], 0)
        self.k_resid[:, :, :r] = K[:, :, Tq:Tk]
        # Values: with the Keys, or (R21) all but the most recent R
        Tqv = Tq if self.v_window == "flush" else max(0, Tk - self.R)
        if Tqv:
            self._store_v(V[:, :, :Tqv], 0)
        self.v_resid[:, :, :Tk - Tqv] = V[:, :, Tqv:Tk]
        self.T = T

    def append(self, k_new: np.ndarray, v_new: np.ndarray):
        """Add one token per sequence ([B, H, d] float16), flushing a full window first."""
        assert self.T + 1 <= self.T_max
        if self.T < self.S:                  # still filling the sink
            self.k_sink[:, :, self.T] = k_new
            self.v_sink[:, :, self.T] = v_new
            self.T += 1
            return
        Tk = self.Tk
        r = self.window_len(Tk)
        token_v = self.v_window == "token"
        if r == self.R:
            # the window is full: its oldest n tokens go to the history (all R of them,
            # reading R5; one Key group, reading R16), the rest move to its front
            n = self.G if self.aging == "group" else self.R
            self._store_k(self.k_resid[:, :, :n], Tk - self.R)
            self.k_resid[:, :, :r - n] = self.k_resid[:, :, n:r].copy()
            if not token_v:
                self._store_v(self.v_resid[:, :, :n], Tk - self.R)
                self.v_resid[:, :, :r - n] = self.v_resid[:, :, n:r].copy()
            r -= n
        self.k_resid[:, :, r] = k_new
        if token_v:
            # R21: a full Value window quantizes its oldest token, then slides
            rv = min(Tk, self.R)
            if rv == self.R:
                self._store_v(self.v_resid[:, :, :1], Tk - self.R)
                self.v_resid[:, :, :rv - 1] = self.v_resid[:, :, 1:rv].copy()
                rv -= 1
            self.v_resid[:, :, rv] = v_new
        else:
            self.v_resid[:, :, r] = v_new
        self.T += 1

    # -- reads ------------------------------------------------------------------------
    def quantized_codes(self):
        """Unpacked codes of the quantized part: k_codes uint8 [B,H,T_q,d] and v_codes
        uint8 [B,H,T_qv,d] (T_qv = T_q unless R21)."""
        Tq, Tqv = self.Tq, self.Tqv
        kc = unpack_keys(self.k_codes[:, :, :Tq], self.bits)
        nrun = (Tqv + V_RUN - 1) // V_RUN
        vc = unpack_values(self.v_codes[:, :, :nrun], self.bits)[:, :, :Tqv]
        return kc, vc

    def dequantized(self):
        """(K_hat, V_hat) float32 [B, H, T, d]: the sink rows, the dequantized history,
        then the residual window."""
        ns = min(self.T, self.S)
        Tq, Tqv = self.Tq, self.Tqv
        r, rv = self.Tk - Tq, self.Tk - Tqv
        kc, vc = self.quantized_codes()
        Kq = dequantize_keys(kc, self.k_scale[:, :, :Tq // self.G],
                             self.k_zero[:, :, :Tq // self.G], self.G)
        Vq = dequantize_values(vc, self.v_scale[:, :, :Tqv], self.v_zero[:, :, :Tqv], self.Gv)
        Kh = np.concatenate([self.k_sink[:, :, :ns].astype(F32), Kq,
                             self.k_resid[:, :, :r].astype(F32)], axis=2)
        Vh = np.concatenate([self.v_sink[:, :, :ns].astype(F32), Vq,
                             self.v_resid[:, :, :rv].astype(F32)], axis=2)
        return Kh, Vh

    def attend(self, q: np.ndarray, sm_scale: float) -> np.ndarray:
        """Decode attention of q [B, H_q, d] float16 over the cache; float32 [B, H_q, d]."""
        Kh, Vh = self.dequantized()
        out = np.empty(q.shape, F32)
        g = q.shape[1] // self.H
        for b in range(self.B):
            for h in range(self.H):
                qs = q[b, h * g:(h + 1) * g]
                out[b, h * g:(h + 1) * g] = attention_fp64(qs, Kh[b, h], Vh[b, h], sm_scale)
        return out


# --------------------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------------------

def attention_fp64(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float) -> np.ndarray:
    """softmax(q K^T * sm_scale) V for queries q [n_q, d] over K, V [T, d]; float64 inside.

    Scaled dot-product attention as written in [INFRA] §2 and [LESTY] §2; the
    ``sm_scale`` float32 value is widened, not recomputed, so both sides use the same
    number.  Returns float32 [n_q, d].
    """
    q64 = q.astype(np.float64)
    K64 = K.astype(np.float64)
    V64 = V.astype(np.float64)
    z = np.float64(F32(sm_scale)) * (q64 @ K64.T)          # [n_q, T]
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    o = (p @ V64) / p.sum(axis=1, keepdims=True)
    return o.astype(F32)


def gqa_attention_fp64(q: np.ndarray, K: np.ndarray, V: np.ndarray,
                       sm_scale: float) -> np.ndarray:
    """Decode attention for all heads: q [B, H_q, d], K/V [B, H_kv, T, d] (reading R6)."""
    B, Hq, d = q.shape
    Hkv = K.shape[1]
    g = Hq // Hkv
    out = np.empty((B, Hq, d), F32)
    for b in range(B):
        for j in range(Hq):
            out[b, j:j + 1] = attention_fp64(q[b, j:j + 1], K[b, j // g], V[b, j // g], sm_scale)
    return out
