#!/usr/bin/env python3
"""Benchmark of the quantized-KV decode path on one MI355X.

One step = one decode step of the streaming hot path on one layer cache: append one
float16 K/V token per sequence (flushing the residual window into the 2/4-bit store
when it is full), then decode attention of the new query over all cached tokens,
through kivi_append_decode (one kernel launch; flush steps add the flush launch, and
so do, with the per-token Value window, steps whose leaving Value completes a 64-token
block of the quantized history).
With --n-split the step is kivi_append_flush + kivi_decode_attn_split.
Steps rotate over ``copies`` independent layer caches (like the layers of a model)
whose total size exceeds the 256 MB last-level cache, so that each step reads its
cache from HBM.  Inputs are resident in HBM before timing starts.

Printed (one JSON line): value = algorithmic bytes of the timed steps / wall time
(GB/s), tokens/s, the decode kernel's roofline against the HBM peak (its algorithmic
bytes per launch over its average duration, from HIP events that the launch itself
records at the kernel's start and end on the launch stream), the CPU oracle's
throughput on a bounded sample, and the output quality against unquantized fp32
attention (reported, not gated).

Algorithmic bytes of a decode launch, per (sequence, KV head): packed codes
T_q*d*b/8 for K and for V, float16 scale+zero 4*d per Key group and 4*(d/G_v) per
token, the float16 residual 2*2*r*d, plus q (2*d per query head) and out (4*d per
query head).  An append adds the new rows (2*2*d read, 2*2*d written) and, when it
flushes, the window read (2*2*R*d) and its codes and scales written.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "quantized-KV decode attention: effective HBM GB/s & % of peak; tokens/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MALL_BYTES = 256 * 2 ** 20
# the decode kernel's sources: its file and the headers it includes
DECODE_SOURCES = tuple(os.path.join(ROOT, "bit_quantization_amd", "csrc", n) for n in
                       ("decode.hip", "decode_common.h", "quantizer.h", "kivi_internal.h"))
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "decode_kernel_hbm_traffic.json")


def source_digest(paths=DECODE_SOURCES):
    """SHA-256 over the decode kernel's source files, in order."""
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per decode launch from the committed PMC record (FETCH_SIZE and
    WRITE_SIZE scaled by a plain copy kernel's reading), or None when the record is
    missing, is for another workload, or the decode source changed since."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get("workloads", {}).get(workload)
    if not entry or rec.get("decode_sources_sha256") != source_digest():
        return None
    return entry.get("traffic_bytes_per_launch")


AGING = "window"     # "group" with --aging group
V_WINDOW = "flush"   # "token" with --v-window token (the per-token Value window)


def window_len(Tk, R, G):
    if Tk == 0:
        return 0
    if AGING == "group":
        return Tk if Tk <= R else R - G + (Tk - R - 1) % G + 1
    return (Tk - 1) % R + 1


def split(T, R, S=0, G=32):
    """(float16 rows, quantized tokens) at T tokens: the first S tokens (the sink) and
    the window of the rest stay float16, the tokens before the window are quantized."""
    ns = min(T, S)
    Tk = T - ns
    r = window_len(Tk, R, G)
    return ns + r, Tk - r


def value_split(T, R, S=0, G=32):
    """(float16 Value rows, quantized Values) at T tokens: as split(), or with the
    per-token Value window the last min(Tk, R) Values in float16."""
    if V_WINDOW != "token":
        return split(T, R, S, G)
    ns = min(T, S)
    Tk = T - ns
    Tqv = max(0, Tk - R)
    return ns + Tk - Tqv, Tqv


class KernelClock:
    """Duration of each timed step's decode kernel itself: before each step the library
    is armed (kivi_time_next_decode) to record a pair of HIP events at that kernel's own
    start and end (hipExtLaunchKernel, on the launch stream), so the dispatch around it
    stays out; the same quantity rocprofv3's kernel trace reports."""

    def __init__(self, n, stream):
        import torch
        self.ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(n)]
        for a, b in self.ev:            # a first record creates the underlying events
            a.record(stream)
            b.record(stream)
        torch.cuda.synchronize()

    def arm(self, i):
        from bit_quantization_amd import kivi as k
        a, b = self.ev[i]
        k.kivi_time_next_decode(a.cuda_event, b.cuda_event)

    def ms(self):
        return [a.elapsed_time(b) for a, b in self.ev]


def decode_bytes(w, T, S=0):
    """Algorithmic bytes of one decode launch at T cached tokens (see module doc)."""
    rows, Tq = split(T, w.residual, S, w.group_k)
    vrows, Tqv = value_split(T, w.residual, S, w.group_k)
    d = w.head_dim
    per_pair = ((Tq + Tqv) * d * w.bits // 8        # K and V codes
                + (Tq // w.group_k) * d * 4         # K scale + zero
                + Tqv * (d // w.group_v) * 4        # V scale + zero
                + (rows + vrows) * d * 2)           # float16 sink + window K and V
    pairs = w.batch * w.kv_heads
    return pairs * per_pair + w.batch * w.q_heads * d * (2 + 4)


def append_bytes(w, T_before, S=0):
    R = w.residual
    d = w.head_dim
    pairs = w.batch * w.kv_heads
    rows = pairs * 2 * d * 2 * 2                    # k_new, v_new read; residual row written
    Tk = T_before - S
    r = 0 if Tk <= 0 else window_len(Tk, R, w.group_k)
    token_v = V_WINDOW == "token"
    if r == R:                                      # flush the window (or its oldest group)
        n = w.group_k if AGING == "group" else R
        nv = 0 if token_v else n                    # Values leave with the Keys, or not
        codes = (n + nv) * d * w.bits // 8
        meta = (n // w.group_k) * d * 4 + nv * (d // w.group_v) * 4
        rows += pairs * ((n + nv) * d * 2 + codes + meta)
    if token_v and Tk >= R:                         # the oldest Value quantized on its own
        rows += pairs * (d * 2 + d * w.bits // 8 + (d // w.group_v) * 4)
    return rows


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="llama8b_128k_2bit",
                   help="workload name (default: the 131072-token shape at 2 bits, the bandwidth target point)")
    p.add_argument("--copies", type=int, default=0, help="layer caches to rotate over (0: auto)")
    p.add_argument("--n-split", type=int, default=0, help="token splits (0: library default)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--sink", type=int, default=0,
                   help="attention-sink tokens kept in float16 at the start of each sequence")
    p.add_argument("--device-lens", action="store_true",
                   help="ragged or paged steps through kivi_append_decode_varlen (the flush "
                        "launch on every step) instead of its host-length variant")
    p.add_argument("--ragged", action="store_true",
                   help="a ragged batch: sequence b holds tokens * (b + 1) / batch tokens")
    p.add_argument("--paged", type=int, default=0, metavar="P",
                   help="a paged cache with pages of P tokens in a shuffled pool (0: contiguous)")
    p.add_argument("--aging", default="window", choices=["window", "group"],
                   help="a full window flushes whole (window) or its oldest Key group (group)")
    p.add_argument("--codec", default="kivi", choices=["kivi", "fp8_e4m3", "fp8_e5m2", "mxfp4"],
                   help="kivi: the workload's 2/4-bit KIVI cache (default); fp8_*: the same "
                        "workload stored as FP8 with per-head scales; mxfp4: stored as MXFP4")
    p.add_argument("--v-window", default="flush", choices=["flush", "token"],
                   help="Values leave the float16 window with the Keys (flush) or one at a "
                        "time (token: KIVI_FLAG_VALUE_TOKEN_WINDOW)")
    p.add_argument("--deterministic", action="store_true",
                   help="KIVI_FLAG_DETERMINISTIC: fixed block order, repeated calls give the "
                        "same output bits")
    p.add_argument("--no-settle", action="store_true",
                   help="no untimed first step per cache (by default each cache takes one, "
                        "which flushes the full window a prompt of a multiple of R leaves)")
    p.add_argument("--no-graph", action="store_true",
                   help="launch the timed steps one by one instead of as one HIP graph")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle sample budget")
    p.add_argument("--read-ceiling", action="store_true",
                   help="time plain reads of the decode working-set sizes (a persistent "
                        "streaming-read kernel) and exit: the rate this GPU reaches at each size")
    p.add_argument("--read-pattern", action="store_true",
                   help="time the 2-bit decode's access pattern without its arithmetic, "
                        "next to a plain read of the same bytes, and exit")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 1 GiB copy kernel (HBM counter calibration)")
    p.add_argument("--timeline", action="store_true",
                   help="per-workgroup clock stamps of the decode kernel (libkivi_timeline.so) "
                        "over back-to-back launches and launches with pauses, then exit")
    return p.parse_args()


def calibrate_copy():
    import torch
    n = 2 ** 30 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)        # one elementwise kernel: reads 1 GiB, writes 1 GiB
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": 2 ** 30, "bytes_written": 2 ** 30,
                      "launches": 5}), flush=True)


# Launch shapes of the plain read (workgroups, threads, loads in flight per lane): one
# persistent workgroup per CU with contiguous shares, and a few neighbours.
READ_SHAPES = ((256, 1024, 8), (256, 512, 8), (256, 512, 16), (256, 1024, 4), (512, 512, 8),
               (1024, 256, 8))
# MiB: the decode step's bytes per launch of each workload (84: 128k 2-bit, 149: 128k
# 4-bit, 172: 32k, 340: 70B stream, 672: one 1M-token layer), then larger reads
READ_SIZES_MB = (84, 149, 172, 340, 672, 1024, 4096)


def probe_library():
    """libkivi_readprobe.so, the benchmark's reference reads (not part of libkivi.so)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "bit_quantization_amd", "libkivi_readprobe.so"))
    P, Z, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.kivi_probe_stream_read.restype = I
    lib.kivi_probe_stream_read.argtypes = [P, Z, I, I, I, P, Z, P, P, P]
    lib.kivi_probe_pattern_read.restype = I
    lib.kivi_probe_pattern_read.argtypes = [P, Z, I, I, I, I, I, P, Z, P, P, P]
    return lib


def read_ceiling():
    """Best-of-5 kernel time of the plain streaming read (libkivi_readprobe.so, a
    bench-only library; HIP events that the launch records at the kernel's own start and
    end, as for the decode's roofline) at the decode working-set sizes, for each launch
    shape in READ_SHAPES; each timed read is of a slice that is not in the 256 MB
    last-level cache."""
    import torch
    lib = probe_library()
    torch.cuda.set_device(0)
    total = 8 << 30
    buf = torch.ones(total // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty(1 << 20, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def read(off, n, shape, ev=(None, None)):
        wg, th, un = shape
        st = lib.kivi_probe_stream_read(buf.data_ptr() + off, n, wg, th, un, sink.data_ptr(),
                                        sink.numel() * 4, stream.cuda_stream, ev[0], ev[1])
        if st != 0:
            raise RuntimeError(f"kivi_probe_stream_read failed ({st})")

    res = {}
    for mb in READ_SIZES_MB:
        n = mb << 20
        slices = total // n
        per = {}
        for shape in READ_SHAPES:
            best = float("inf")
            for rep in range(5):
                s0 = ((rep * 3 + 1) % slices) * n
                # a 1 GiB read of another part first: it keeps the GPU busy while the timed
                # interval is enqueued and leaves the last-level cache without the slice
                o = (((s0 >> 30) + 4) % (total >> 30)) << 30
                read(o, 1 << 30, (256, 1024, 8))
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)            # creates the events; the launch records them
                b.record(stream)
                read(s0, n, shape, (a.cuda_event, b.cuda_event))
                torch.cuda.synchronize()
                best = min(best, a.elapsed_time(b) / 1e3)
            per["x".join(map(str, shape))] = round(best * 1e6, 2)
        key = min(per, key=per.get)
        t = per[key] / 1e6
        res[f"{mb}MB"] = {"best_shape": key, "us": per[key], "GB/s": round(n / t / 1e9, 1),
                          "pct_of_peak": round(100 * n / t / 1e9 / HBM_PEAK_GBS, 1),
                          "us_by_shape": per}
        print(f"[read] {mb} MB: {res[f'{mb}MB']}", file=sys.stderr, flush=True)
    print(json.dumps({"read_ceiling": res,
                      "kernel": "stream_read_kernel (persistent: workgroups x threads x loads "
                                "in flight per lane, contiguous share per workgroup)",
                      "timing": "kernel start/end events (hipExtLaunchKernel), best of 5"}),
          flush=True)


# One decode step's quantized blocks at two workload shapes (the history's whole 64-token
# blocks; the float16 window holds the rest): (workload, pairs, blocks per pair,
# workgroups per pair as the decode plans them)
PATTERN_SHAPES = (("llama8b_32k", 64, 510, 4), ("llama8b_128k_2bit", 8, 2046, 32))


def read_pattern():
    """The 2-bit decode's access pattern without its arithmetic (libkivi_readprobe.so,
    kivi_probe_pattern_read): the bytes of one decode step of each PATTERN_SHAPES shape
    (5376 B per 64-token block), read with the decode kernel's lane offsets from the six
    arrays of the cache layout, or contiguously per block, with 1 to 3 blocks in flight per
    wave; beside it the plain read of the same byte count (best launch shape of
    READ_SHAPES).  Best-of-5 kernel-event times, each of a slice outside the last-level
    cache after a 1 GiB read of another part."""
    import torch
    lib = probe_library()
    torch.cuda.set_device(0)
    total = 8 << 30
    buf = torch.ones(total // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty(1 << 20, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def timed(n, launch):
        slices = total // n
        best = float("inf")
        for rep in range(5):
            s0 = ((rep * 3 + 1) % slices) * n
            o = (((s0 >> 30) + 4) % (total >> 30)) << 30
            if lib.kivi_probe_stream_read(buf.data_ptr() + o, 1 << 30, 256, 1024, 8,
                                          sink.data_ptr(), sink.numel() * 4,
                                          stream.cuda_stream, None, None):
                raise RuntimeError("kivi_probe_stream_read failed")
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            b.record(stream)
            st = launch(buf.data_ptr() + s0, a.cuda_event, b.cuda_event)
            if st != 0:
                raise RuntimeError(f"probe launch failed ({st})")
            torch.cuda.synchronize()
            best = min(best, a.elapsed_time(b) / 1e3)
        return best * 1e6

    res = {}
    for name, pairs, blocks, nw in PATTERN_SHAPES:
        n = pairs * blocks * 5376
        plain = {}
        for wg, th, un in READ_SHAPES:
            plain["x".join(map(str, (wg, th, un)))] = round(timed(n, lambda p, e0, e1: (
                lib.kivi_probe_stream_read(p, n, wg, th, un, sink.data_ptr(), sink.numel() * 4,
                                           stream.cuda_stream, e0, e1))), 2)
        best_plain = min(plain.values())
        modes = {}
        for fused in (0, 1):
            for ahead in (1, 2, 3):
                key = f"{'fused_blocks' if fused else 'six_arrays'}_ahead{ahead}"
                modes[key] = round(timed(n, lambda p, e0, e1: (
                    lib.kivi_probe_pattern_read(p, n, pairs, blocks, nw, ahead, fused,
                                                sink.data_ptr(), sink.numel() * 4,
                                                stream.cuda_stream, e0, e1))), 2)
        res[name] = {"pairs": pairs, "blocks_per_pair": blocks, "workgroups_per_pair": nw,
                     "bytes": n, "plain_read_us": best_plain, "plain_read_by_shape": plain,
                     "pattern_us": modes,
                     "pattern_over_plain": {k: round(v / best_plain, 3) for k, v in modes.items()}}
        print(f"[pattern] {name}: plain {best_plain} us, {modes}", file=sys.stderr, flush=True)
    print(json.dumps({"read_pattern": res,
                      "kernel": "pattern_read_kernel (2-bit decode lane offsets, 8 waves per "
                                "workgroup, a ring of register sets) and stream_read_kernel",
                      "timing": "kernel start/end events (hipExtLaunchKernel), best of 5"}),
          flush=True)


def timeline(args):
    """Where one decode launch's time goes and at what clock: the timeline build of the
    library (libkivi_timeline.so, the same sources with KIVI_TIMELINE) has every workgroup
    stamp the 100 MHz real-time counter and the shader clock counter when it starts, when
    its blocks are done, when its arrival is counted and, in the last arriver, when its
    own partial stores are complete, when the first round of partial loads is complete
    and when the merge is done.  On the workload's layer caches (rotated as in the
    benchmark) it runs 64 warmup launches, then three series of 64: back to back, with
    5 ms pauses, back to back.  Per launch: the span from the first start to the last
    event, the start spread, blocks done (first / median / last workgroup), arrival and
    merge times, all from the first start; a workgroup's own stream time (start to blocks
    done, median over workgroups); the last arrivers' median phases (arrival to own stores
    complete, to partial loads complete, to merge done); and the median over workgroups
    of the shader clock while streaming (clock-counter ticks over real-time ticks between
    start and blocks done).  --n-split sets the workgroups per (sequence, KV head) pair
    (at most one per 64-token block plus one).  Prints one JSON line of medians and
    per-launch series."""
    import ctypes

    import numpy as np
    ROOT_LIB = os.path.join(ROOT, "bit_quantization_amd", "libkivi_timeline.so")
    os.environ["KIVI_LIBRARY"] = ROOT_LIB         # read by the binding at import
    import torch

    import workloads as W
    from bit_quantization_amd import kivi as k
    if os.path.realpath(k.LIB_PATH) != os.path.realpath(ROOT_LIB):
        raise RuntimeError("the timeline mode needs the binding to load libkivi_timeline.so")
    lib = ctypes.CDLL(ROOT_LIB)
    geo = (ctypes.c_int(), ctypes.c_int(), ctypes.c_int())
    lib.kivi_timeline_geometry(*[ctypes.byref(x) for x in geo])
    NS, NWG, NM = (x.value for x in geo)
    torch.cuda.set_device(0)
    w = W.get(args.workload).replace(layers=1)
    dims = k.Dims(1, w.batch, w.kv_heads, w.q_heads, w.head_dim, w.bits, w.group_k,
                  w.group_v, w.residual, w.max_tokens() + 64)
    per_copy = decode_bytes(w, w.tokens + 1)
    copies = args.copies or max(2, math.ceil(4 * MALL_BYTES / per_copy))
    caches = []
    for c in range(copies):
        K, V = W.make_kv(w, c, device="cuda", total_tokens=w.tokens + 2)
        cache = k.Cache(dims)
        k.kivi_quantize_k(dims, cache, 0, K, w.tokens + 1, K.shape[2])
        k.kivi_quantize_v(dims, cache, 0, V, w.tokens + 1, V.shape[2])
        caches.append(cache)
        del K, V
    q = W.make_q(w, 0, 0, device="cuda")
    out = torch.empty((w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    T = w.tokens + 1
    ws = k.new_workspace(dims, T, args.n_split)
    n_split = args.n_split or k.kivi_decode_splits(dims, T)
    nwg = w.batch * w.kv_heads * n_split
    if nwg > NWG:
        raise RuntimeError(f"{nwg} workgroups: the timeline build stamps at most {NWG}")
    buf = np.zeros(NS * NWG * NM * 2, dtype=np.uint64)

    def launch(i):
        k.kivi_decode_attn(dims, caches[i % copies], 0, T, q, w.sm_scale, out, ws,
                           n_split=args.n_split)

    def phase(rt, merged, m0, m1):
        # median over a launch's last arrivers of the time from mark m0 to mark m1
        if NM <= max(m0, m1) or not merged.any():
            return None
        return float(np.median(rt[merged, m1] - rt[merged, m0])) / 100.0

    def series(pause):
        for i in range(NS):
            launch(i)
            if pause:
                torch.cuda.synchronize()
                time.sleep(pause)
        torch.cuda.synchronize()
        if lib.kivi_timeline_read(buf.ctypes.data_as(ctypes.c_void_p), ctypes.c_size_t(buf.nbytes)):
            raise RuntimeError("kivi_timeline_read failed")
        A = buf.reshape(NS, NWG, NM, 2).astype(np.int64)[:, :nwg]
        rows = []
        for sl in range(NS):
            a = A[sl]
            rt = a[:, :, 0]
            t0 = rt[:, 0].min()
            us = lambda x: (x - t0) / 100.0
            merged = rt[:, 3] > 0
            arrived = rt[:, 2] > 0
            end = max(rt[:, 1].max(), rt[arrived, 2].max() if arrived.any() else 0,
                      rt[merged, 3].max() if merged.any() else 0)
            clk = np.median((a[:, 1, 1] - a[:, 0, 1]) / np.maximum(rt[:, 1] - rt[:, 0], 1) * 100.0)
            rows.append({"span_us": us(end), "start_spread_us": us(rt[:, 0].max()),
                         "blocks_done_first_us": us(rt[:, 1].min()),
                         "blocks_done_median_us": float(np.median(us(rt[:, 1]))),
                         "blocks_done_last_us": us(rt[:, 1].max()),
                         "workgroup_stream_median_us": float(np.median(rt[:, 1] - rt[:, 0])) / 100.0,
                         "arrival_median_us": (float(np.median(us(rt[arrived, 2])))
                                               if arrived.any() else None),
                         "arrival_last_us": us(rt[arrived, 2].max()) if arrived.any() else None,
                         "merge_done_last_us": us(rt[merged, 3].max()) if merged.any() else None,
                         "merger_stores_us": phase(rt, merged, 2, 4),
                         "merger_loads_us": phase(rt, merged, 4, 5),
                         "merger_fold_us": phase(rt, merged, 5, 3),
                         "clock_mhz": float(clk)})
        return rows

    # clear the stamps of earlier launches, then warm up
    for i in range(NS):
        launch(i)
    torch.cuda.synchronize()
    res = {"timeline": args.workload, "workgroups": nwg, "n_split": n_split,
           "layer_caches": copies, "series": {}}
    for name, pause in (("back_to_back", 0), ("paused_5ms", 0.005), ("back_to_back_2", 0)):
        rows = series(pause)
        med = {key: round(float(np.median([r[key] for r in rows if r[key] is not None])), 2)
               for key in rows[0]}
        res["series"][name] = {"median": med,
                               "span_us": [round(r["span_us"], 2) for r in rows],
                               "clock_mhz": [round(r["clock_mhz"]) for r in rows]}
        print(f"[timeline] {name}: {med}", file=sys.stderr, flush=True)
    print(json.dumps(res), flush=True)


def prefill_bytes(w, T, S=0):
    """Algorithmic bytes of quantizing one layer's prompt of T tokens (a1 + a2): read
    fp16 K and V, write codes, scales/zeros and the fp16 sink and window rows."""
    rows, Tq = split(T, w.residual, S, w.group_k)
    d = w.head_dim
    per_pair = (2 * T * d * 2                           # K and V read
                + 2 * Tq * d * w.bits // 8              # codes written
                + (Tq // w.group_k) * d * 4 + Tq * (d // w.group_v) * 4
                + 2 * rows * d * 2)                     # float16 rows written
    return w.batch * w.kv_heads * per_pair


def cpu_baseline(w, host_pairs, budget_s, S=0):
    """Time the CPU oracle's decode step (append + attend) on a bounded sample.

    A few (sequence, KV head) pairs of the workload are prefilled (untimed); then
    consecutive decode steps (append the next token, attend over the cache) run
    round-robin over those pairs until ``budget_s`` seconds of oracle time are used.
    """
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    one = w.replace(batch=1, kv_heads=1, q_heads=w.gqa)
    caches = []
    for (Kh, Vh, k_rows, v_rows, qh, T) in host_pairs:
        m = math.lcm(16, w.group_k, w.residual)
        cap = (T + len(k_rows) + 1 + m - 1) // m * m
        oc = O.LayerCache(1, 1, w.head_dim, w.bits, w.group_k, w.group_v, w.residual, cap,
                          sink=S, aging=AGING, v_window=V_WINDOW)
        oc.prefill(Kh, Vh)
        caches.append((oc, k_rows, v_rows, qh))
    done_bytes, t_used, steps, T_last = 0, 0.0, 0, 0
    j = 0
    while t_used < budget_s:
        oc, k_rows, v_rows, qh = caches[steps % len(caches)]
        j = steps // len(caches)
        if j >= len(k_rows):
            break
        T = oc.T
        t0 = time.perf_counter()
        oc.append(k_rows[j][None, None], v_rows[j][None, None])
        oc.attend(qh, w.sm_scale)
        t_used += time.perf_counter() - t0
        done_bytes += decode_bytes(one, T + 1, S) + append_bytes(one, T, S)
        steps += 1
        T_last = T + 1
    return {"value": done_bytes / t_used / 1e9, "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"{steps} oracle decode steps (append + attend, {w.gqa} query heads, "
                       f"~{T_last} tokens) round-robin over {len(caches)} (sequence, KV head) "
                       f"pairs of the workload, {t_used:.1f} s of oracle time; "
                       f"os.cpu_count()={os.cpu_count()}, BLAS threads={threads}")}


def fp8_decode_bytes(w, T):
    """Algorithmic bytes of one FP8 decode launch at T tokens: per (sequence, KV head)
    T*d Key and T*d Value code bytes and 8 bytes of scales; q and out per query head."""
    d = w.head_dim
    return w.batch * w.kv_heads * (2 * T * d + 8) + w.batch * w.q_heads * d * (2 + 4)


def fp8_append_bytes(w):
    """k_new, v_new read (2 * 2d) and their codes written (2d), per (sequence, KV head)."""
    return w.batch * w.kv_heads * (2 * 2 * w.head_dim + 2 * w.head_dim)


def mx_decode_bytes(w, T):
    """Algorithmic bytes of one MXFP4 decode launch at T tokens: per (sequence, KV head)
    and token d/2 Key and d/2 Value code bytes and d/32 scale bytes each; q and out."""
    d = w.head_dim
    return w.batch * w.kv_heads * T * 2 * (d // 2 + d // 32) + w.batch * w.q_heads * d * (2 + 4)


def mx_append_bytes(w):
    """k_new, v_new read (2 * 2d) and their codes and scales written."""
    d = w.head_dim
    return w.batch * w.kv_heads * (2 * 2 * d + 2 * (d // 2 + d // 32))


def fp8_cpu_baseline(w, fmt, host_pairs, budget_s):
    """The FP8 oracle's decode step (append + attend) on a bounded sample, as
    cpu_baseline."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    one = w.replace(batch=1, kv_heads=1, q_heads=w.gqa)
    caches = []
    mx = fmt == "mxfp4"
    for (Kh, Vh, k_rows, v_rows, qh, T, ks, vs) in host_pairs:
        cap = (T + len(k_rows) + 1 + 31) // 32 * 32
        oc = (O.MXFP4Cache(1, 1, w.head_dim, cap) if mx
              else O.FP8Cache(1, 1, w.head_dim, fmt, cap, ks, vs))
        oc.prefill(Kh, Vh)
        caches.append((oc, k_rows, v_rows, qh))
    done_bytes, t_used, steps, T_last = 0, 0.0, 0, 0
    while t_used < budget_s:
        oc, k_rows, v_rows, qh = caches[steps % len(caches)]
        j = steps // len(caches)
        if j >= len(k_rows):
            break
        T = oc.T
        t0 = time.perf_counter()
        oc.append(k_rows[j][None, None], v_rows[j][None, None])
        oc.attend(qh, w.sm_scale)
        t_used += time.perf_counter() - t0
        done_bytes += (mx_decode_bytes(one, T + 1) + mx_append_bytes(one) if mx
                       else fp8_decode_bytes(one, T + 1) + fp8_append_bytes(one))
        steps += 1
        T_last = T + 1
    return {"value": done_bytes / t_used / 1e9, "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"{steps} {'MXFP4' if mx else 'FP8'} oracle decode steps (append + attend, {w.gqa} query heads, "
                       f"~{T_last} tokens) round-robin over {len(caches)} (sequence, KV head) "
                       f"pairs of the workload, {t_used:.1f} s of oracle time; "
                       f"os.cpu_count()={os.cpu_count()}, BLAS threads={threads}")}


def fp8_main(args):
    """The workload stored as FP8 (one step = kivi_fp8_append + kivi_fp8_decode_attn) or
    as MXFP4 (kivi_mxfp4_append + kivi_mxfp4_decode_attn)."""
    import numpy as np
    import torch

    import workloads as W
    from bit_quantization_amd import kivi as k

    mx = args.codec == "mxfp4"
    fmt = "mxfp4" if mx else args.codec[4:]
    dec_bytes = mx_decode_bytes if mx else fp8_decode_bytes
    app_bytes = mx_append_bytes if mx else fp8_append_bytes
    torch.cuda.set_device(0)
    w = W.get(args.workload)
    w1 = w.replace(layers=1) if w.layers > 1 else w
    total_steps = args.warmup + 2 * args.steps
    per_copy = dec_bytes(w1, w1.tokens)
    copies = args.copies or max(1, math.ceil(4 * MALL_BYTES / per_copy))
    if w.layers > 1:
        copies = args.copies or min(w.layers, max(copies, 2))
    steps_per_copy = math.ceil(total_steps / copies) + 1
    extra = max(steps_per_copy, 1024)
    Tmax = (w1.tokens + steps_per_copy + 31) // 32 * 32
    dims = (k.MxDims(1, w1.batch, w1.kv_heads, w1.q_heads, w1.head_dim, Tmax) if mx
            else k.Fp8Dims(1, w1.batch, w1.kv_heads, w1.q_heads, w1.head_dim, fmt, Tmax))
    print(f"[bench] workload {w.name} as {args.codec}: {copies} layer caches x "
          f"{per_copy / 1e6:.1f} MB decode reads, {args.warmup}+{args.steps} steps",
          file=sys.stderr, flush=True)
    top = 448.0 if fmt == "e4m3" else 57344.0
    caches, Ts, news, host_pairs = [], [], [], []
    rng = np.random.default_rng(0)
    sample = [(int(b), int(h)) for b, h in zip(rng.integers(0, w1.batch, 6),
                                               rng.integers(0, w1.kv_heads, 6))]
    for c in range(copies):
        K, V = W.make_kv(w1, c, device="cuda", total_tokens=w1.tokens + extra)
        # per-head scales from the largest magnitude of the prompt: a calibration on the
        # synthetic data ("4.4 KV Cache quantization" §4.2, calibrated scales)
        ks = (K[:, :, :w1.tokens].float().abs().amax(dim=(0, 2, 3)) / top).clamp_min(1e-12)
        vs = (V[:, :, :w1.tokens].float().abs().amax(dim=(0, 2, 3)) / top).clamp_min(1e-12)
        if mx:                  # MXFP4 needs no calibration: every block has its own scale
            cache = k.MxCache(dims)
            k.kivi_mxfp4_quantize(dims, cache, 0, K, V, w1.tokens, K.shape[2])
        else:
            cache = k.Fp8Cache(dims, ks.cpu(), vs.cpu())
            k.kivi_fp8_quantize(dims, cache, 0, K, V, w1.tokens, K.shape[2])
        caches.append(cache)
        Ts.append(w1.tokens)
        news.append((K[:, :, w1.tokens:w1.tokens + steps_per_copy].permute(2, 0, 1, 3).contiguous(),
                     V[:, :, w1.tokens:w1.tokens + steps_per_copy].permute(2, 0, 1, 3).contiguous()))
        if c == 0 and not args.no_cpu_baseline:
            q0 = W.make_q(w1, 0, 0, device="cuda").cpu().numpy()
            g = w1.gqa
            for (b, h) in sample:
                host_pairs.append((K[b:b + 1, h:h + 1, :w1.tokens].cpu().numpy(),
                                   V[b:b + 1, h:h + 1, :w1.tokens].cpu().numpy(),
                                   K[b, h, w1.tokens:].cpu().numpy(), V[b, h, w1.tokens:].cpu().numpy(),
                                   q0[b:b + 1, h * g:(h + 1) * g], w1.tokens,
                                   float(ks[h]), float(vs[h])))
        del K, V
    qs = [W.make_q(w1, 0, s_, device="cuda") for s_ in range(8)]
    out = torch.empty((w1.batch, w1.q_heads, w1.head_dim), dtype=torch.float32, device="cuda")
    ws = (k.new_mxfp4_workspace if mx else k.new_fp8_workspace)(dims, Tmax, args.n_split)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def prepare(i):
        c = i % copies
        T_before = Ts[c]
        j = T_before - w1.tokens
        kn, vn = news[c]
        T = T_before + 1
        Ts[c] = T
        q = qs[i % len(qs)]

        if mx and not args.n_split:
            call = k.prepare_mxfp4_step(dims, caches[c], 0, T_before, kn[j], vn[j], q,
                                        w1.sm_scale, out, ws)
        elif mx:
            def call(c=c, T_before=T_before, T=T, kj=kn[j], vj=vn[j], q=q):
                k.kivi_mxfp4_append(dims, caches[c], 0, T_before, kj, vj)
                k.kivi_mxfp4_decode_attn(dims, caches[c], 0, T, q, w1.sm_scale, out, ws,
                                         args.n_split)
        else:
            def call(c=c, T_before=T_before, T=T, kj=kn[j], vj=vn[j], q=q):
                k.kivi_fp8_append(dims, caches[c], 0, T_before, kj, vj)
                k.kivi_fp8_decode_attn(dims, caches[c], 0, T, q, w1.sm_scale, out, ws,
                                       args.n_split)
        return call, dec_bytes(w1, T), app_bytes(w1)

    for i in range(args.warmup):
        prepare(i)[0]()
    torch.cuda.synchronize()
    clock = KernelClock(args.steps, stream)
    steps = [prepare(args.warmup + i) for i in range(args.steps)]
    # the decode kernel's bytes: the MXFP4 step's decode also codes the new token; the
    # FP8 step's append is a launch of its own
    one_launch = mx and not args.n_split
    launch_bytes = sum(db + (ab if one_launch else 0) for _, db, ab in steps)
    torch.cuda.synchronize()
    for i, (call, _, _) in enumerate(steps):
        clock.arm(i)
        call()
    torch.cuda.synchronize()
    ms = clock.ms()
    avg_s = sum(ms) / len(ms) / 1e3
    first = args.warmup + args.steps
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        steps = [prepare(first + i) for i in range(args.steps)]
        for call, _, _ in steps:
            call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del graph
    total = sum(db + ab for _, db, ab in steps)
    value = total / wall / 1e9
    achieved = launch_bytes / args.steps / avg_s / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        cpu = fp8_cpu_baseline(w1, fmt, host_pairs, args.cpu_seconds)
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp4+f16+f32" if mx else "fp8+f16+f32",
        "data": "synthetic (seeded N(0,1) K/V/Q with x50 Key outlier channels and x100 Value "
                "outlier tokens; " + ("MXFP4 block scales from the data)" if mx else
                                      "per-head FP8 scales from the prompt's largest magnitude)"),
        "config": {"workload": w.name, "codec": args.codec, "batch": w1.batch,
                   "kv_heads": w1.kv_heads, "q_heads": w1.q_heads, "head_dim": w1.head_dim,
                   "tokens": w1.tokens, "layer_caches": copies,
                   "step": ("kivi_mxfp4_append + kivi_mxfp4_decode_attn" if mx
                            else "kivi_fp8_append + kivi_fp8_decode_attn"),
                   "launch": "one HIP graph of the timed steps"},
        "tokens_per_s": round(w1.batch * args.steps / wall, 1),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "kernel": ("mx_decode_kernel (append fused)" if one_launch
                                                else "mx_decode_kernel" if mx
                                                else "fp8_decode_kernel"),
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "bytes_per_launch": int(launch_bytes / args.steps),
                     "avg_launch_us": round(avg_s * 1e6, 3),
                     "median_launch_us": round(sorted(ms)[len(ms) // 2] * 1e3, 3),
                     "p10_p90_launch_us": [round(sorted(ms)[len(ms) // 10] * 1e3, 3),
                                           round(sorted(ms)[(9 * len(ms)) // 10] * 1e3, 3)],
                     "timing": "decode kernel start/end events (kivi_time_next_decode)",
                     "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this path has no "
              f"multi-GPU mode", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.read_ceiling:
        read_ceiling()
        return
    if args.read_pattern:
        read_pattern()
        return
    if args.timeline:
        timeline(args)
        return
    if args.codec != "kivi":
        fp8_main(args)
        return

    import numpy as np
    import torch

    import workloads as W
    from bit_quantization_amd import kivi as k

    torch.cuda.set_device(0)
    w = W.get(args.workload)
    if w.layers != 1:
        # multi-layer workload: every layer is one cache of the rotation
        w1 = w.replace(layers=1)
    else:
        w1 = w
    S = args.sink
    global AGING, V_WINDOW
    AGING = args.aging
    V_WINDOW = args.v_window
    one = w1.replace(batch=1)
    # prompt length of each sequence: all w1.tokens, or tokens * (b + 1) / batch
    base = [w1.tokens * (b + 1) // w1.batch if args.ragged else w1.tokens
            for b in range(w1.batch)]

    def step_bytes(T_before):
        """(decode bytes, append bytes) of the step that appends at T_before + j."""
        return (sum(decode_bytes(one, t + 1, S) for t in T_before),
                sum(append_bytes(one, t, S) for t in T_before))

    per_copy_bytes = step_bytes(base)[0]
    copies = args.copies or max(1, math.ceil(4 * MALL_BYTES / per_copy_bytes))
    if w.layers > 1:
        copies = args.copies or min(w.layers, max(copies, 2))
    # one settling step per cache, the warmup, the eager loop timed per launch (roofline),
    # then the K steps of the graph
    settle = 0 if args.no_settle else copies
    total_steps = settle + args.warmup + 2 * args.steps
    steps_per_copy = math.ceil(total_steps / copies) + 1
    extra_rows = max(steps_per_copy, 1024)          # rows appended on the GPU / by the oracle
    Tmax = w1.replace(stream_steps=steps_per_copy).max_tokens()
    dims = k.Dims(1, w1.batch, w1.kv_heads, w1.q_heads, w1.head_dim, w1.bits, w1.group_k,
                  w1.group_v, w1.residual, Tmax, sink=S, aging=AGING,
                  v_window=V_WINDOW, deterministic=args.deterministic)
    print(f"[bench] workload {w.name}: {copies} layer caches x {per_copy_bytes / 1e6:.1f} MB "
          f"decode reads, {args.warmup}+{args.steps} steps", file=sys.stderr, flush=True)

    caches, Ts, news = [], [], []
    keep = None
    host_pairs = []
    rng = np.random.default_rng(0)
    sample_pairs = [(int(b), int(h)) for b, h in zip(rng.integers(0, w1.batch, 64),
                                                      rng.integers(0, w1.kv_heads, 64))]
    T_hi = max(base)
    base_t = torch.tensor(base, dtype=torch.int32, device="cuda")
    varlen = args.ragged or args.paged > 0
    paging = None
    if args.paged:
        # every sequence's pages drawn from one shuffled pool (a seeded permutation)
        per_seq = -(-Tmax // args.paged)
        perm = np.random.default_rng(0).permutation(w1.batch * per_seq).astype(np.int32)
        paging = k.Paging(args.paged, per_seq, w1.batch * per_seq,
                          torch.from_numpy(perm.reshape(w1.batch, per_seq)).cuda())

    def new_cache():
        return k.PagedCache(dims, paging) if paging else k.Cache(dims)
    # per-sequence token counts before step j of a copy (ragged calls read them on the GPU;
    # the host copy lets a step without a flush skip the flush launch)
    lens_steps = torch.stack([base_t + j for j in range(steps_per_copy)]).contiguous()
    lens_host = None if args.device_lens else lens_steps.cpu()

    def rows_from(X, j0, n):
        """X[b, :, base[b] + j0 + t] for t < n, as [n, B, H, d] (contiguous per step)."""
        return torch.stack([X[b, :, base[b] + j0:base[b] + j0 + n] for b in range(w1.batch)]) \
            .permute(2, 0, 1, 3).contiguous()

    for c in range(copies):
        K, V = W.make_kv(w1, c, device="cuda", total_tokens=w1.tokens + extra_rows)
        cache = new_cache()
        if varlen:
            k.kivi_quantize_k_varlen(dims, cache, 0, K, base_t, T_hi, K.shape[2], paging=paging)
            k.kivi_quantize_v_varlen(dims, cache, 0, V, base_t, T_hi, V.shape[2], paging=paging)
        else:
            k.kivi_quantize_k(dims, cache, 0, K, w1.tokens, K.shape[2])
            k.kivi_quantize_v(dims, cache, 0, V, w1.tokens, V.shape[2])
        caches.append(cache)
        Ts.append(0)                                # steps taken on this copy
        news.append((rows_from(K, 0, steps_per_copy), rows_from(V, 0, steps_per_copy)))
        if c == 0:
            keep = (K, V)
            if not args.no_cpu_baseline:
                q0 = W.make_q(w1, 0, 0, device="cuda").cpu().numpy()
                g = w1.gqa
                for (b, h) in sample_pairs[:6]:
                    t = base[b]
                    host_pairs.append((K[b:b + 1, h:h + 1, :t].cpu().numpy(),
                                       V[b:b + 1, h:h + 1, :t].cpu().numpy(),
                                       K[b, h, t:].cpu().numpy(), V[b, h, t:].cpu().numpy(),
                                       q0[b:b + 1, h * g:(h + 1) * g], t))
        else:
            del K, V
    qs = [W.make_q(w1, 0, s, device="cuda") for s in range(8)]
    out = torch.empty((w1.batch, w1.q_heads, w1.head_dim), dtype=torch.float32, device="cuda")
    ws = k.new_workspace(dims, Tmax, args.n_split)
    n_split = args.n_split or k.kivi_decode_splits(dims, T_hi)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    flushes = {}                                    # step i -> does it flush a window

    def prepare(i):
        """Step i: one decode step (append the token, flushing a full window, then
        attend), with its arguments marshalled now so that the timed loops only make
        the calls; one kernel launch except on flush steps (1 in R), which add the
        flush launch.  Returns (call, decode bytes, append bytes)."""
        c = i % copies
        j = Ts[c]
        Ts[c] = j + 1
        # steps with the append launch before the decode: a full window flushes, or
        # (per-token Value window) the Value leaving the window completes a 64-token
        # block of the quantized history (the decode quantizes it itself otherwise)
        def two_launch(Tk, R=w1.residual):
            if Tk <= 0:
                return False
            if window_len(Tk, R, w1.group_k) == R:
                return True
            return V_WINDOW == "token" and Tk >= R and (Tk - R + 1) % 64 == 0
        flushes[i] = any(two_launch(t + j - S) for t in base)
        T_before = T_hi + j                         # the longest sequence's count
        T = T_before + 1
        kn, vn = news[c]
        q = qs[i % len(qs)]
        db, ab = step_bytes([t + j for t in base])
        if varlen:
            call = k.prepare_append_decode_varlen(
                dims, caches[c], 0, lens_steps[j], T_before, kn[j], vn[j], q, w1.sm_scale, out,
                ws, paging=paging, T_before_host=None if lens_host is None else lens_host[j])
        elif args.n_split:
            def call(c=c, T_before=T_before, T=T, kj=kn[j], vj=vn[j], q=q):
                k.kivi_append_flush(dims, caches[c], 0, T_before, kj, vj)
                k.kivi_decode_attn(dims, caches[c], 0, T, q, w1.sm_scale, out, ws,
                                   n_split=args.n_split)
        else:
            call = k.prepare_append_decode(dims, caches[c], 0, T_before, kn[j], vn[j], q,
                                           w1.sm_scale, out, ws)
        return call, db, ab

    # Settling: every cache takes its first decode step untimed.  A prompt whose length is
    # a multiple of R leaves the float16 window full, so that step flushes it; the timed
    # steps then see the steady state, where one step in R flushes (those first steps'
    # launch times are reported as roofline.settle_steps).
    settle_ms, settle_flush = [], 0
    for i in range(settle):
        call = prepare(i)[0]
        settle_flush += flushes[i]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        e1.synchronize()
        settle_ms.append(e0.elapsed_time(e1))
    for i in range(settle, settle + args.warmup):
        prepare(i)[0]()
    torch.cuda.synchronize()

    # Duration of the dominant kernel (roofline): K eager steps; the decode kernel of
    # each is timed by events at its own start and end (KernelClock).
    t_first = settle + args.warmup
    clock = KernelClock(args.steps, stream)
    steps = [prepare(t_first + i) for i in range(args.steps)]
    # the decode kernel's bytes: a one-launch step's decode also appends (and, with the
    # per-token Value window, quantizes the leaving Value); a two-launch step's append
    # kernel does that instead, except in ragged steps, whose decode stores every new row
    kernel_bytes = [db + (0 if (flushes[t_first + i] and not varlen) or args.n_split else ab)
                    for i, (_, db, ab) in enumerate(steps)]
    torch.cuda.synchronize()
    for i, (call, _, _) in enumerate(steps):
        clock.arm(i)
        call()
    torch.cuda.synchronize()
    dec_ms = clock.ms()
    # decode-kernel times of steps with two launches (a window flush first) and of the
    # others
    kinds = {}
    for name, want in (("flush", True), ("plain", False)):
        idx = [i for i in range(len(dec_ms)) if flushes[t_first + i] == want]
        if idx:
            kinds[name] = {"steps": len(idx),
                           "avg_kernel_us": round(sum(dec_ms[i] for i in idx) / len(idx) * 1e3, 3)}
    dec_avg_s = sum(dec_ms) / len(dec_ms) / 1e3
    dec_med_s = sorted(dec_ms)[len(dec_ms) // 2] / 1e3
    dec_per_launch = sum(kernel_bytes) / args.steps

    # Whole-job throughput: the next K steps, launched as one HIP graph (captured with
    # each step's own arguments, so replaying it once runs exactly those K steps and
    # the host's per-call cost leaves the timed region), between two synchronizations.
    first = t_first + args.steps
    if args.no_graph:
        steps = [prepare(first + i) for i in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for call, _, _ in steps:
            call()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    else:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            # the calls are marshalled inside the capture: they must use its stream
            steps = [prepare(first + i) for i in range(args.steps)]
            for call, _, _ in steps:
                call()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        del graph
    wall = t1 - t0
    dec_bytes = sum(db for _, db, _ in steps)
    app_bytes = sum(ab for _, _, ab in steps)

    # Quality versus unquantized fp32 attention on copy 0 (reported, not gated).
    K, V = keep
    quality = None
    if not varlen:
        Tq = w1.tokens + Ts[0]
        qq = qs[0]
        k.kivi_decode_attn(dims, caches[0], 0, Tq, qq, w1.sm_scale, out, ws,
                           n_split=args.n_split)
        g = w1.gqa
        Kf = K[:, :, :Tq].float()
        Vf = V[:, :, :Tq].float()
        qf = qq.float().view(w1.batch, w1.kv_heads, g, w1.head_dim)
        logits = torch.matmul(qf, Kf.transpose(-1, -2).contiguous()) * float(np.float32(w1.sm_scale))
        ref = torch.matmul(torch.softmax(logits, dim=-1), Vf).view_as(out)
        o = out.double()
        rd = ref.double()
        quality = {"vs": "unquantized fp32 attention on the same float16 K/V",
                   "rel_l2": float((o - rd).norm() / rd.norm()),
                   "cosine": float(torch.nn.functional.cosine_similarity(o.flatten(),
                                                                         rd.flatten(), dim=0)),
                   "max_abs": float((o - rd).abs().max())}
        del Kf, Vf
    del K, V, keep

    # Secondary: prefill quantization (a1 + a2) of one layer's prompt, re-run on
    # copy 0's fp16 K/V into a scratch cache (HIP events, best of 3).
    Kp, Vp = W.make_kv(w1, 0, device="cuda", total_tokens=T_hi)
    scratch = new_cache()
    pre_s = float("inf")
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        if varlen:
            k.kivi_quantize_k_varlen(dims, scratch, 0, Kp, base_t, T_hi, Kp.shape[2],
                                     paging=paging)
            k.kivi_quantize_v_varlen(dims, scratch, 0, Vp, base_t, T_hi, Vp.shape[2],
                                     paging=paging)
        else:
            k.kivi_quantize_k(dims, scratch, 0, Kp, w1.tokens, Kp.shape[2])
            k.kivi_quantize_v(dims, scratch, 0, Vp, w1.tokens, Vp.shape[2])
        b.record()
        b.synchronize()
        pre_s = min(pre_s, a.elapsed_time(b) / 1e3)
    del Kp, Vp, scratch
    pre_bytes = sum(prefill_bytes(one, t, S) for t in base)
    prefill = {"what": "kivi_quantize_k + kivi_quantize_v of one layer's prompt",
               "tokens": sum(base), "us": round(pre_s * 1e6, 1),
               "GB/s": round(pre_bytes / pre_s / 1e9, 1), "bytes": pre_bytes}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w1, host_pairs, args.cpu_seconds, S)

    total_bytes = dec_bytes + app_bytes
    value = total_bytes / wall / 1e9
    achieved = dec_per_launch / dec_avg_s / 1e9
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8+f32",
        "data": "synthetic (seeded N(0,1) K/V/Q with x50 Key outlier channels and x100 Value "
                "outlier tokens; no dataset or weights)",
        "config": {"workload": w.name, "batch": w1.batch, "kv_heads": w1.kv_heads,
                   "q_heads": w1.q_heads, "head_dim": w1.head_dim, "tokens": w1.tokens,
                   "bits": w1.bits, "group_k": w1.group_k, "group_v": w1.group_v,
                   "residual": w1.residual, "sink": S, "aging": AGING, "v_window": V_WINDOW,
                   "deterministic": args.deterministic,
                   "lengths": ("tokens * (b + 1) / batch: " + ",".join(map(str, base))
                               if args.ragged else "uniform"),
                   "paged": (f"pages of {args.paged} tokens, shuffled pool" if args.paged
                             else "contiguous"),
                   "layer_caches": copies,
                   "n_split": n_split,
                   "step": "append(+flush) + decode attention" + (
                       "" if not varlen else
                       "; lengths on the device only: flush launch every step"
                       if args.device_lens else
                       "; lengths also on the host: flush launch on flush steps only"),
                   "launch": "one HIP graph of the timed steps" if not args.no_graph
                             else "one call per step"},
        "tokens_per_s": round(w1.batch * args.steps / wall, 1),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm",
                     "kernel": "decode_kernel (append fused; work queue + merge)",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "bytes_per_launch": int(dec_per_launch),
                     "avg_launch_us": round(dec_avg_s * 1e6, 3),
                     "median_launch_us": round(dec_med_s * 1e6, 3),
                     "p10_p90_launch_us": [round(sorted(dec_ms)[len(dec_ms) // 10] * 1e3, 3),
                                           round(sorted(dec_ms)[(9 * len(dec_ms)) // 10] * 1e3, 3)],
                     "timing": "decode kernel start/end events (kivi_time_next_decode)",
                     "traffic": measured_traffic(w.name)
                                if S == 0 and AGING == "window" and V_WINDOW == "flush"
                                and not varlen else None,
                     "step_kinds": kinds,
                     # the first settling step also carries the process's first launch
                     # of each kernel (its code object is loaded then), so it is
                     # reported apart from the others
                     "settle_steps": ({"steps": settle, "flush_steps": settle_flush,
                                       "first_us": round(settle_ms[0] * 1e3, 3),
                                       "others_avg_us": (round(sum(settle_ms[1:]) /
                                                               (settle - 1) * 1e3, 3)
                                                         if settle > 1 else None)}
                                      if settle else None)},
        "cpu_baseline": cpu,
        "prefill_quantize": prefill,
        "quality": quality,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
