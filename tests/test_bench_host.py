"""Host-side accounting of bench.py (CPU only): the window rule it uses to split
tokens, the algorithmic bytes of a decode launch and of an append, and which steps
flush, checked against the oracle's own definitions (oracle/kivi_ref.py)."""
import importlib.util
import os

import pytest

import oracle as O
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_host", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture
def bench():
    return load_bench()


@pytest.mark.parametrize("R,G", [(128, 32), (32, 32), (64, 16)])
def test_window_rule_matches_oracle(bench, R, G):
    bench.AGING = "window"
    for T in range(0, 5 * R + 3):
        assert bench.window_len(T, R, G) == O.residual_len(T, R)
    bench.AGING = "group"
    for T in range(0, 5 * R + 3):
        assert bench.window_len(T, R, G) == O.residual_len_grouped(T, R, G)


@pytest.mark.parametrize("name", ["tiny", "llama8b_32k", "llama8b_128k_4bit",
                                  "llama8b_128k_2bit", "llama70b_stream", "long_1m"])
def test_decode_bytes_are_the_cache_plus_q_and_out(bench, name):
    """A decode launch reads the whole cache of one layer (codes, scales, zeros, the
    float16 window) once, each query once and writes each output once."""
    bench.AGING = "window"
    w = W.get(name).replace(layers=1)
    for T in (w.tokens, w.tokens + 1, w.tokens + w.residual):
        cache = O.kivi_cache_bytes(1, w.batch, T, w.kv_heads, w.head_dim, w.bits, w.group_k,
                                   w.group_v, w.residual)["total"]
        q_out = w.batch * w.q_heads * w.head_dim * (2 + 4)
        assert bench.decode_bytes(w, T) == cache + q_out


def test_decode_bytes_per_token_and_head(bench):
    """84 bytes per quantized token and KV head at 2 bits, 148 at 4 bits (G = 32,
    G_v = 128, d = 128), 512 per float16 token."""
    bench.AGING = "window"
    for bits, per_tok in ((2, 84), (4, 148)):
        w = W.get("tiny").replace(bits=bits, batch=1, kv_heads=1, q_heads=1)
        T0, T1 = 257, 257 + 128                   # same window length (1 token)
        assert bench.decode_bytes(w, T1) - bench.decode_bytes(w, T0) == 128 * per_tok


def test_flush_steps_of_the_70b_stream(bench):
    """Of 256 appends from 32768 tokens (R = 128), those at T_before = 32768 and
    32896 flush the window: exactly the appends whose byte count includes a flush."""
    bench.AGING = "window"
    w = W.get("llama70b_stream").replace(layers=1)
    plain = bench.append_bytes(w, w.tokens + 1)
    flushing = [j for j in range(256) if bench.append_bytes(w, w.tokens + j) != plain]
    assert flushing == [0, 128]
    for j in range(256):
        r = O.residual_len(w.tokens + j, w.residual)
        assert (j in flushing) == (r == w.residual)


@pytest.mark.parametrize("aging", ["window", "group"])
def test_decode_bytes_with_the_token_value_window(bench, aging):
    """With the per-token Value window the decode reads the Key history and window as
    before and the Values split at the oracle's T_qv: codes and scales of the quantized
    Values, float16 rows of the rest."""
    bench.AGING, bench.V_WINDOW = aging, "token"
    try:
        w = W.get("tiny").replace(residual=64)
        d, b = w.head_dim, w.bits
        for T in (1, 63, 64, 65, 100, 257, 1000):
            oc = O.LayerCache(1, 1, d, b, w.group_k, w.group_v, w.residual, 1024, aging=aging,
                              v_window="token")
            oc.T = T                                    # only the split rule is used
            Tq, Tqv = oc.Tq, oc.Tqv
            r, rv = oc.Tk - Tq, oc.Tk - Tqv
            ref = ((Tq + Tqv) * d * b // 8 + (Tq // w.group_k) * d * 4 + Tqv * 4
                   + (r + rv) * d * 2 + w.q_heads * d * 6)
            assert bench.decode_bytes(w, T) == ref, T
    finally:
        bench.AGING, bench.V_WINDOW = "window", "flush"
