"""The seeded input generators: shapes, determinism and the outlier recipe."""
import numpy as np
import pytest
import torch

import workloads as W


def test_every_workload_is_consistent():
    for w in W.WORKLOADS.values():
        assert w.q_heads % w.kv_heads == 0 and w.gqa in (1, 2, 4, 8)
        assert w.residual % w.group_k == 0 and w.residual % 16 == 0
        m = w.max_tokens()
        assert m > w.total_tokens and m % 16 == 0 and m % w.group_k == 0 and m % w.residual == 0


def test_make_kv_is_deterministic_and_injects_outliers():
    w = W.get("tiny").replace(batch=2, kv_heads=2, q_heads=4, tokens=400)
    K1, V1 = W.make_kv(w, 0)
    K2, V2 = W.make_kv(w, 0)
    assert K1.dtype == torch.float16 and K1.shape == (2, 2, 400, 128)
    assert torch.equal(K1, K2) and torch.equal(V1, V2)
    K3, _ = W.make_kv(w, 1)
    assert not torch.equal(K1, K3)
    k_ch, v_tok = W.outlier_indices(w, 0)
    assert k_ch.shape == (2, 4) and v_tok.shape == (2, 2)
    Kf, Vf = K1.float(), V1.float()
    for h in range(2):
        ch_rms = Kf[:, h].pow(2).mean(dim=(0, 1)).sqrt()
        top = set(torch.topk(ch_rms, 4).indices.tolist())
        assert top == set(k_ch[h].tolist())
        assert float(ch_rms[k_ch[h]].min()) > 20 * float(ch_rms.median())
    for b in range(2):
        tok_rms = Vf[b].pow(2).mean(dim=(0, 2)).sqrt()
        sel = v_tok[b][v_tok[b] >= 0]
        assert set(torch.topk(tok_rms, len(sel)).indices.tolist()) == set(sel.tolist())


def test_one_percent_value_outliers_plus_token_zero():
    w = W.get("llama8b_32k")
    k_ch, v_tok = W.outlier_indices(w, 0)
    assert v_tok.shape == (8, 327 + 1)
    assert np.all(v_tok[:, 0] == 0)
    assert all(len(set(r.tolist())) == len(r) for r in v_tok)
    s = W.get("llama70b_stream")
    assert W.outlier_indices(s, 0)[1].shape == (16, int(0.01 * 33024) + 1)


def test_queries_differ_per_step():
    w = W.get("tiny")
    assert not torch.equal(W.make_q(w, 0, 0), W.make_q(w, 0, 1))
    assert torch.equal(W.make_q(w, 0, 3), W.make_q(w, 0, 3))
