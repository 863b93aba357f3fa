"""Write tests/golden/quality_report.json: the quality of the quantized cache, computed
by the CPU oracle only (reported, not a pass/fail bar).

For one (sequence, KV head) pair of each workload shape (the workload reduced to one
sequence and one KV head with its query heads, drawn by workloads.make_kv on the CPU:
the same recipe and outlier channels as the GPU runs, other normal draws), the decode
output of
  * KIVI: Keys per channel over groups of G tokens, Values per token (oracle LayerCache),
  * the ablation with per-token Keys: Keys quantized like Values (groups of G_v
    channels of one token), everything else unchanged,
is compared with float64 attention over the original float16 K/V: relative L2 error,
cosine and largest absolute error of the outputs, and the relative error of the
dequantized Keys on the ordinary channels and on the x50 outlier channels.
"KV Cache Quantization (KIVI & FP4)" §6.5 and "KIVI: A Tuning-Free Asymmetric 2bit
Quantization for KV Cache" ("Keys and values are not the same animal"): a per-token Key
scale is set by the outlier channels, so the ordinary channels lose their resolution.

Run from the repository root: python tests/golden/make_quality_report.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O          # noqa: E402
import workloads as W       # noqa: E402

OUT = os.path.join(ROOT, "tests", "golden", "quality_report.json")
F32 = np.float32


def pair_quality(w, T=None):
    """Metrics for layer 0 of workload w reduced to one (sequence, KV head) pair."""
    T = T or w.tokens
    w = w.replace(batch=1, kv_heads=1, q_heads=w.gqa, layers=1)
    b = h = 0
    K, V = W.make_kv(w.replace(layers=1), 0, device="cpu", total_tokens=T)
    q = W.make_q(w, 0, 0, device="cpu").numpy()
    g = w.gqa
    Kh = K[b:b + 1, h:h + 1].numpy()
    Vh = V[b:b + 1, h:h + 1].numpy()
    qh = q[b:b + 1, h * g:(h + 1) * g]
    m = int(np.lcm.reduce([16, w.group_k, w.residual]))
    cap = (T + 1 + m - 1) // m * m
    oc = O.LayerCache(1, 1, w.head_dim, w.bits, w.group_k, w.group_v, w.residual, cap)
    oc.prefill(Kh, Vh)
    ref = O.attention_fp64(qh[0], Kh[0, 0], Vh[0, 0], w.sm_scale).astype(np.float64)
    kivi = oc.attend(qh, w.sm_scale)[0].astype(np.float64)
    Kq, Vq = oc.dequantized()                      # per-channel Keys, per-token Values
    # the ablation: the quantized Key history coded per token instead
    Tq = oc.Tq
    kc, ks, kz = O.quantize_values(Kh[0, 0, :Tq], w.group_v, w.bits)
    Kt = np.concatenate([O.dequantize_values(kc, ks, kz, w.group_v),
                         Kh[0, 0, Tq:].astype(F32)], axis=0)
    tok = O.attention_fp64(qh[0], Kt, Vq[0, 0], w.sm_scale).astype(np.float64)
    k_ch, _ = W.outlier_indices(w.replace(layers=1), 0, T)
    out_ch = np.zeros(w.head_dim, bool)
    out_ch[k_ch[h]] = True
    K0 = Kh[0, 0, :Tq].astype(np.float64)

    def k_err(Khat, mask):
        e = Khat[:Tq][:, mask].astype(np.float64) - K0[:, mask]
        return float(np.linalg.norm(e) / np.linalg.norm(K0[:, mask]))

    def out_metrics(o):
        return {"rel_l2": float(np.linalg.norm(o - ref) / np.linalg.norm(ref)),
                "cosine": float((o * ref).sum() / np.linalg.norm(o) / np.linalg.norm(ref)),
                "max_abs": float(np.abs(o - ref).max())}

    return {
        "tokens": T, "quantized_tokens": Tq, "bits": w.bits, "query_heads": g,
        "kivi_per_channel_keys": {**out_metrics(kivi),
                                  "key_rel_err_ordinary_channels": k_err(Kq[0, 0], ~out_ch),
                                  "key_rel_err_outlier_channels": k_err(Kq[0, 0], out_ch)},
        "ablation_per_token_keys": {**out_metrics(tok),
                                    "key_rel_err_ordinary_channels": k_err(Kt, ~out_ch),
                                    "key_rel_err_outlier_channels": k_err(Kt, out_ch)},
    }


def main():
    report = {"what": __doc__.split("\n\n")[0],
              "pairs": "each workload reduced to one sequence and one KV head, layer 0",
              "data": "workloads.make_kv on the CPU (seeded; N(0,1), x50 Key channels, x100 "
                      "Value tokens), query workloads.make_q step 0",
              "workloads": {}}
    for name in ("tiny", "llama8b_32k", "llama8b_128k_2bit", "llama8b_128k_4bit",
                 "llama70b_stream"):
        w = W.get(name)
        report["workloads"][name] = pair_quality(w)
        print(name, json.dumps(report["workloads"][name]), flush=True)
    with open(OUT, "w") as f:
        json.dump(report, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
