"""Seeded synthetic workloads shared by the tests, the benchmark and the oracle checks.

This module only *draws inputs*. It holds none of the quantization or attention
arithmetic, so both the CPU oracle and the GPU path can consume what it produces
without sharing any of the method's code.

The shapes follow the model shapes the pages quote (Llama-3-8B / Llama-3-70B
layers: 8 KV heads, head_dim 128, GQA 4:1 and 8:1; "KV Cache Quantization (KIVI &
FP4)" §1 and "09 — KV Cache Quantization", "The number that motivates
everything"). The outlier structure follows "09 — KV Cache Quantization", "The
structural fact that makes KV quant work": a few Key channels are tens of times
larger than the rest for every token, and a few Value tokens are hundreds of times
larger than the median. No dataset, checkpoint or evaluation item is used.

Recipe (identical for every workload):
  * K, V are drawn as float32 N(0, 1) and Q as float32 N(0, 1).
  * Key outlier channels: per KV head (shared by every sequence of the batch),
    ``k_outlier_channels`` distinct channels are multiplied by ``k_outlier_scale``
    for every token.
  * Value outlier tokens: per sequence (shared by every KV head),
    ``v_outlier_tokens(T)`` distinct token positions are multiplied by
    ``v_outlier_scale`` for every channel.
  * The float32 tensors are rounded to float16 (round-to-nearest-even).
  * Indices of outliers come from ``numpy.random.default_rng(seed)``; the normal
    draws come from ``torch.Generator(device).manual_seed(seed)`` so that large
    layers can be drawn directly in device memory.  The same tensor is then handed
    to both sides (copied to host for the oracle).
  * Seeds: ``1000 * workload.seed_id + layer`` for K/V, ``+ 500 + step`` offset
    streams for Q (see :func:`make_q`).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get", "make_kv", "make_q", "outlier_indices"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed_id: int
    layers: int
    batch: int
    kv_heads: int
    q_heads: int
    head_dim: int
    tokens: int              # cached tokens at the decode step (after prefill)
    bits: int
    group_k: int             # G: tokens per Key group
    group_v: int             # G_v: channels per Value group
    residual: int            # R: fp16 residual window
    k_outlier_channels: int = 4
    k_outlier_scale: float = 50.0
    v_outlier_scale: float = 100.0
    v_outlier_frac: float = 0.01    # fraction of tokens with outlier Values
    v_outlier_count: Optional[int] = None  # fixed count instead of a fraction
    v_outlier_include_token0: bool = True
    stream_steps: int = 0    # decode steps appended after prefill (streaming mode)
    description: str = ""

    @property
    def gqa(self) -> int:
        return self.q_heads // self.kv_heads

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def total_tokens(self) -> int:
        """Tokens drawn for K/V: prefill plus every streamed step."""
        return self.tokens + self.stream_steps

    def v_outlier_tokens(self, total_tokens: int) -> int:
        if self.v_outlier_count is not None:
            return self.v_outlier_count
        return int(math.floor(self.v_outlier_frac * total_tokens))

    def max_tokens(self) -> int:
        """Capacity of the cache: every token ever appended, rounded up to 16 and R."""
        need = self.total_tokens + 1
        step = math.lcm(16, self.residual, self.group_k)
        return ((need + step - 1) // step) * step

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of the headline metric plus the 2-bit variant of the 131072-token
# shape, which is the bandwidth target point.
WORKLOADS = {
    "tiny": Workload(
        name="tiny", seed_id=1, layers=1, batch=1, kv_heads=1, q_heads=1, head_dim=128,
        tokens=256, bits=2, group_k=32, group_v=128, residual=32,
        v_outlier_count=2, v_outlier_include_token0=False,
        description="1 layer, B=1, 1 KV head, 1 query head, d=128, T=256, 2-bit, G=32, "
                    "G_v=128, R=32; 4 K channels x50, 2 V tokens x100"),
    "llama8b_32k": Workload(
        name="llama8b_32k", seed_id=2, layers=1, batch=8, kv_heads=8, q_heads=32, head_dim=128,
        tokens=32768, bits=2, group_k=32, group_v=128, residual=128,
        description="Llama-3-8B-shaped layer: B=8, 32 query / 8 KV heads, d=128, T=32768, "
                    "2-bit, G=32, R=128"),
    "llama8b_128k_4bit": Workload(
        name="llama8b_128k_4bit", seed_id=3, layers=1, batch=1, kv_heads=8, q_heads=32,
        head_dim=128, tokens=131072, bits=4, group_k=32, group_v=128, residual=128,
        description="Llama-3-8B-shaped layer at 4-bit: B=1, T=131072, G=32, R=128"),
    "llama8b_128k_2bit": Workload(
        name="llama8b_128k_2bit", seed_id=6, layers=1, batch=1, kv_heads=8, q_heads=32,
        head_dim=128, tokens=131072, bits=2, group_k=32, group_v=128, residual=128,
        description="the 131072-token shape at 2-bit (bandwidth target point)"),
    "llama70b_stream": Workload(
        name="llama70b_stream", seed_id=4, layers=1, batch=16, kv_heads=8, q_heads=64,
        head_dim=128, tokens=32768, bits=2, group_k=32, group_v=128, residual=128,
        stream_steps=256,
        description="Llama-3-70B-shaped layer, streaming: B=16, 64 query / 8 KV heads, "
                    "prefill 32768 then 256 append+decode steps, 2-bit, G=32, R=128"),
    "long_1m": Workload(
        name="long_1m", seed_id=5, layers=32, batch=1, kv_heads=8, q_heads=32, head_dim=128,
        tokens=1048576, bits=2, group_k=32, group_v=128, residual=128,
        v_outlier_count=2, v_outlier_include_token0=False,
        description="32 layers x 8 KV heads x d=128, T=1048576, 2-bit, G=32, R=128, "
                    "one decode step across all layers"),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def outlier_indices(w: Workload, layer: int, total_tokens: Optional[int] = None):
    """Return (k_channels [H_kv, n_ch], v_tokens [B, n_tok]) as int64 numpy arrays."""
    T = w.total_tokens if total_tokens is None else total_tokens
    rng = np.random.default_rng(1000 * w.seed_id + layer)
    k_ch = np.stack([
        rng.choice(w.head_dim, size=w.k_outlier_channels, replace=False)
        for _ in range(w.kv_heads)
    ]).astype(np.int64)
    n_tok = min(w.v_outlier_tokens(T), T)
    rows = []
    for _ in range(w.batch):
        if w.v_outlier_include_token0 and T > 0:
            pick = rng.choice(np.arange(1, T), size=min(n_tok, T - 1), replace=False) if T > 1 \
                else np.zeros(0, np.int64)
            pick = np.concatenate([[0], pick])
        else:
            pick = rng.choice(T, size=n_tok, replace=False)
        rows.append(np.sort(pick).astype(np.int64))
    width = max((len(r) for r in rows), default=0)
    v_tok = np.full((w.batch, width), -1, np.int64)
    for b, r in enumerate(rows):
        v_tok[b, :len(r)] = r
    return k_ch, v_tok


def make_kv(w: Workload, layer: int = 0, device="cpu", total_tokens: Optional[int] = None):
    """Draw K and V for one layer as float16 torch tensors [B, H_kv, T, d].

    ``total_tokens`` defaults to prefill + streamed tokens.  Draws happen in float32
    on ``device`` and are rounded to float16 there.
    """
    import torch

    T = w.total_tokens if total_tokens is None else total_tokens
    gen = torch.Generator(device=device)
    gen.manual_seed(1000 * w.seed_id + layer)
    shape = (w.batch, w.kv_heads, T, w.head_dim)
    k = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    v = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    k_ch, v_tok = outlier_indices(w, layer, T)
    for h in range(w.kv_heads):
        idx = torch.as_tensor(k_ch[h], device=device)
        k[:, h, :, idx] *= w.k_outlier_scale
    for b in range(w.batch):
        sel = v_tok[b][v_tok[b] >= 0]
        if len(sel):
            idx = torch.as_tensor(sel, device=device)
            v[b, :, idx, :] *= w.v_outlier_scale
    return k.to(torch.float16), v.to(torch.float16)


def make_q(w: Workload, layer: int = 0, step: int = 0, device="cpu"):
    """Draw one decode query [B, H_q, d] float16 for ``step`` (fresh per step)."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(1000 * w.seed_id + 500 + 7919 * layer + step)
    q = torch.randn((w.batch, w.q_heads, w.head_dim), generator=gen, device=device,
                    dtype=torch.float32)
    return q.to(torch.float16)
