"""GPU parity of paged caches: the quantized history of every sequence lives in pages
of P tokens taken from a pool in the order a block table gives (here a seeded
shuffle, so neighbouring history tokens sit in distant pages).

Paging is layout only: the oracle is one oracle cache per sequence, and each
sequence's pages, read back in block-table order, must hold its oracle history
bytes exactly; attention within |gpu - ref| <= 2e-3 + 1e-3 |ref|.
"""
import math

import numpy as np
import pytest

import workloads as W
from tests.test_gpu_parity import assert_close, rand_kv
from tests.test_gpu_ragged import lens_tensor, seq_oracle
from tests.test_gpu_sink import capacity, compare_sink_cache, sink_dims

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

D = 128
HISTORY = ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero")


def kv():
    from bit_quantization_amd import kivi
    return kivi


def make_paging(dims, P, seed, spare=3):
    """Every sequence gets its own pages, drawn from a shuffled pool with spare pages."""
    per_seq = -(-dims.max_tokens // P)
    n = dims.batch * per_seq + spare
    perm = np.random.default_rng(seed).permutation(n)[:dims.batch * per_seq]
    table = torch.from_numpy(perm.reshape(dims.batch, per_seq).astype(np.int32)).cuda()
    return kv().Paging(P, per_seq, n, table)


class SequenceView:
    """One sequence of a paged cache seen as a one-sequence contiguous cache."""

    def __init__(self, cache, b):
        self.cache, self.b, self.dims = cache, b, cache.dims

    def view(self, name):
        if name in HISTORY:
            return self.cache.sequence_view(name, 0, self.b)[None, None]
        return self.cache.view(name)[:, self.b:self.b + 1]


def paged_prefill(dims, paging, K, V, lens):
    k = kv()
    cache = k.PagedCache(dims, paging)
    T_hi = max(lens)
    lt = lens_tensor(lens)
    k.kivi_quantize_k_varlen(dims, cache, 0, K, lt, T_hi, K.shape[2], paging=paging)
    k.kivi_quantize_v_varlen(dims, cache, 0, V, lt, T_hi, V.shape[2], paging=paging)
    return cache


def check_sequences(cache, K, V, lens):
    torch.cuda.synchronize()
    for b, T in enumerate(lens):
        compare_sink_cache(SequenceView(cache, b), seq_oracle(cache.dims, K, V, b, T), T, seq=0)


CASES = [
    # bits, G, R, S, aging, P, lens
    (2, 32, 128, 0, "window", 128, [1000, 37, 129, 256, 1, 0]),
    (4, 64, 128, 4, "window", 64, [700, 3, 131, 1301]),
    (2, 32, 128, 0, "group", 256, [1000, 129, 97, 161]),
    (4, 32, 64, 7, "group", 128, [7, 300, 72, 0]),
]


@pytest.mark.parametrize("bits,G,R,S,aging,P,lens", CASES)
def test_paged_prefill_is_bit_exact(bits, G, R, S, aging, P, lens):
    B, H = len(lens), 2
    T_hi = max(lens)
    dims = sink_dims(bits, G, 128, R, S, B, H, 1, capacity(T_hi, R), aging)
    paging = make_paging(dims, P, seed=T_hi)
    K, V = rand_kv(B, H, T_hi + 2, D, seed=P + B)
    check_sequences(paged_prefill(dims, paging, K, V, lens), K, V, lens)


@pytest.mark.parametrize("bits,G,R,S,aging,P,lens", CASES[:3])
def test_paged_appends_equal_per_sequence_prefill(bits, G, R, S, aging, P, lens):
    k = kv()
    B, H = len(lens), 2
    steps = R + 2 * G + 3
    T_end = max(lens) + steps
    dims = sink_dims(bits, G, 128, R, S, B, H, 1, capacity(T_end, R), aging)
    paging = make_paging(dims, P, seed=steps)
    K, V = rand_kv(B, H, T_end, D, seed=steps + P)
    cache = paged_prefill(dims, paging, K, V, lens)
    cur = list(lens)
    for _ in range(steps):
        kn = torch.stack([K[b, :, cur[b]] for b in range(B)]).contiguous()
        vn = torch.stack([V[b, :, cur[b]] for b in range(B)]).contiguous()
        k.kivi_append_flush_varlen(dims, cache, 0, lens_tensor(cur), max(cur), kn, vn,
                                   paging=paging)
        cur = [t + 1 for t in cur]
    check_sequences(cache, K, V, cur)


DECODE = [
    # bits, G, R, S, aging, P, g, lens
    (2, 32, 128, 0, "window", 128, 4, [1000, 37, 129, 256, 1, 2048]),
    (4, 64, 128, 4, "window", 64, 2, [700, 3, 4, 131, 1301]),
    (2, 32, 128, 0, "group", 256, 8, [1000, 129, 97, 161]),
    (4, 32, 64, 7, "group", 128, 1, [7, 3000, 72]),
    # one long sequence whose pairs merge in several rounds
    (2, 32, 128, 0, "window", 128, 4, [20000, 100]),
]


@pytest.mark.parametrize("bits,G,R,S,aging,P,g,lens", DECODE)
def test_paged_decode_matches_oracle(bits, G, R, S, aging, P, g, lens):
    k = kv()
    B, H = len(lens), 2
    T_hi = max(lens)
    dims = sink_dims(bits, G, 128, R, S, B, H, g, capacity(T_hi, R), aging)
    paging = make_paging(dims, P, seed=g)
    K, V = rand_kv(B, H, T_hi, D, seed=T_hi + P, scale=3.0)
    K[:, :, :, 17] *= 30
    cache = paged_prefill(dims, paging, K, V, lens)
    gq = torch.Generator(device="cuda")
    gq.manual_seed(P + g)
    q = torch.randn((B, H * g, D), generator=gq, device="cuda").to(torch.float16)
    out = torch.empty((B, H * g, D), dtype=torch.float32, device="cuda")
    sm = 1 / math.sqrt(D)
    k.kivi_decode_attn_varlen(dims, cache, 0, lens_tensor(lens), T_hi, q, sm, out,
                              k.new_workspace(dims, T_hi), paging=paging)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b, T in enumerate(lens):
        ref = seq_oracle(dims, K, V, b, T).attend(q[b:b + 1].cpu().numpy(), sm)
        assert_close(got[b:b + 1], ref, f"paged decode sequence {b} T={T}")


@pytest.mark.parametrize("S,aging", [(0, "window"), (5, "group")])
@pytest.mark.parametrize("host", [False, True])
def test_paged_append_decode_equals_contiguous(host, S, aging):
    # the fused ragged step on a paged cache against the same steps on a contiguous
    # cache: outputs to float32 rounding, every sequence's history bytes identical.
    # host: the paged side steps through kivi_append_decode_varlen_host (a host copy of
    # the counts; the flush launch only on the steps where some window is full)
    k = kv()
    bits, G, R, g, P = 2, 32, 64, 4, 64
    lens = [2, 70, 63, 64, 200]
    B, H = len(lens), 2
    steps = R + G + 4
    T_end = max(lens) + steps
    dims = sink_dims(bits, G, 128, R, S, B, H, g, capacity(T_end, R), aging)
    paging = make_paging(dims, P, seed=9)
    K, V = rand_kv(B, H, T_end, D, seed=21)
    a = paged_prefill(dims, paging, K, V, lens)
    b_ = k.Cache(dims)
    lt0 = lens_tensor(lens)
    k.kivi_quantize_k_varlen(dims, b_, 0, K, lt0, max(lens), K.shape[2])
    k.kivi_quantize_v_varlen(dims, b_, 0, V, lt0, max(lens), V.shape[2])
    wa, wb = k.new_workspace(dims, T_end), k.new_workspace(dims, T_end)
    oa = torch.empty((B, H * g, D), dtype=torch.float32, device="cuda")
    ob = torch.empty_like(oa)
    gq = torch.Generator(device="cuda")
    gq.manual_seed(3)
    cur = list(lens)
    for step in range(steps):
        q = torch.randn((B, H * g, D), generator=gq, device="cuda").to(torch.float16)
        lt = lens_tensor(cur)
        kn = torch.stack([K[b, :, cur[b]] for b in range(B)]).contiguous()
        vn = torch.stack([V[b, :, cur[b]] for b in range(B)]).contiguous()
        k.kivi_append_decode_varlen(dims, a, 0, lt, max(cur), kn, vn, q, 0.09, oa, wa,
                                    paging=paging,
                                    T_before_host=torch.tensor(cur, dtype=torch.int32)
                                    if host else None)
        k.kivi_append_decode_varlen(dims, b_, 0, lt, max(cur), kn, vn, q, 0.09, ob, wb)
        torch.cuda.synchronize()
        assert np.allclose(oa.cpu().numpy(), ob.cpu().numpy(), rtol=1e-5, atol=1e-6), step
        cur = [t + 1 for t in cur]
    for b, T in enumerate(cur):
        oc = seq_oracle(dims, K, V, b, T)
        Tq = oc.Tq
        got = a.sequence_view("k_codes", 0, b)[:, :Tq].cpu().numpy()
        assert np.array_equal(got, b_.view("k_codes")[0, b, :, :Tq].cpu().numpy())
        if S == 0:
            assert np.array_equal(got, oc.k_codes[0, :, :Tq])
    check_sequences(a, K, V, cur)


def test_paged_out_of_range_table_entries_stay_inside_the_pool():
    # a table entry outside [0, pages) is clamped on the device: the call completes and
    # the sequences with valid tables are unaffected
    k = kv()
    lens = [300, 200]
    B, H, g = 2, 1, 2
    dims = sink_dims(2, 32, 128, 128, 0, B, H, g, capacity(300, 128))
    paging = make_paging(dims, 64, seed=4)
    K, V = rand_kv(B, H, 300, D, seed=8)
    cache = paged_prefill(dims, paging, K, V, lens)
    bad = paging.block_table.clone()
    bad[1, 0] = -7
    bad[1, 1] = 1 << 30
    bad_paging = k.Paging(paging.page_tokens, paging.pages_per_seq, paging.pages, bad)
    gq = torch.Generator(device="cuda")
    gq.manual_seed(2)
    q = torch.randn((B, H * g, D), generator=gq, device="cuda").to(torch.float16)
    out = torch.empty((B, H * g, D), dtype=torch.float32, device="cuda")
    k.kivi_decode_attn_varlen(dims, cache, 0, lens_tensor(lens), 300, q, 0.1, out,
                              k.new_workspace(dims, 300), paging=bad_paging)
    torch.cuda.synchronize()
    ref = seq_oracle(dims, K, V, 0, 300).attend(q[0:1].cpu().numpy(), 0.1)
    assert_close(out[0:1].cpu().numpy(), ref, "sequence with a valid table")


def test_paged_workload_8b_length_mix_sampled():
    # the 8B-shaped 32k workload as a ragged paged batch (4k .. 32k tokens, pages of
    # 128 tokens in a shuffled pool); sampled pairs recomputed by the oracle
    k = kv()
    w = W.get("llama8b_32k")
    print("[parity] paged workload llama8b_32k 4k..32k P=128", flush=True)
    lens = [4096 * (b + 1) for b in range(w.batch)]
    T_hi = max(lens)
    dims = k.Dims(1, w.batch, w.kv_heads, w.q_heads, w.head_dim, w.bits, w.group_k, w.group_v,
                  w.residual, w.max_tokens())
    paging = make_paging(dims, 128, seed=1)
    Kd, Vd = W.make_kv(w, 0, device="cuda", total_tokens=T_hi)
    cache = paged_prefill(dims, paging, Kd, Vd, lens)
    q = W.make_q(w, 0, 0, device="cuda")
    out = torch.empty((w.batch, w.q_heads, D), dtype=torch.float32, device="cuda")
    k.kivi_decode_attn_varlen(dims, cache, 0, lens_tensor(lens), T_hi, q, w.sm_scale, out,
                              k.new_workspace(dims, T_hi), paging=paging)
    torch.cuda.synchronize()
    g = w.gqa
    one = k.Dims(1, 1, 1, g, w.head_dim, w.bits, w.group_k, w.group_v, w.residual,
                 w.max_tokens())
    for b, h in [(0, 1), (4, 4), (7, 6)]:
        T = lens[b]
        oc = seq_oracle(one, Kd[:, h:h + 1], Vd[:, h:h + 1], b, T)
        Tq = oc.Tq
        got = cache.sequence_view("k_codes", 0, b)[h, :Tq].cpu().numpy()
        assert np.array_equal(got, oc.k_codes[0, 0, :Tq])
        ref = oc.attend(q[b:b + 1, h * g:(h + 1) * g].cpu().numpy(), w.sm_scale)
        assert_close(out[b, h * g:(h + 1) * g].cpu().numpy(), ref[0], f"paged pair {(b, h)} T={T}")
