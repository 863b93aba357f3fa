"""The quality report (tests/golden/quality_report.json, written by
tests/golden/make_quality_report.py from the oracle alone): reported numbers, with the
qualitative claim the pages make checked here.  Per-channel Key groups keep the ordinary
channels' resolution when a few channels are x50 outliers; per-token Key groups do not
("KV Cache Quantization (KIVI & FP4)" §6.5; "KIVI: A Tuning-Free Asymmetric 2bit
Quantization for KV Cache", "Keys and values are not the same animal")."""
import importlib.util
import json
import os

import pytest

from tests.conftest import ROOT

REPORT = os.path.join(ROOT, "tests", "golden", "quality_report.json")


def load_script():
    spec = importlib.util.spec_from_file_location(
        "quality_report", os.path.join(ROOT, "tests", "golden", "make_quality_report.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name,bits", [("llama8b_32k", 2), ("llama8b_128k_4bit", 4)])
def test_per_channel_keys_beat_per_token_keys(name, bits):
    import workloads as W
    mod = load_script()
    q = mod.pair_quality(W.get(name), T=2048)
    kivi, tok = q["kivi_per_channel_keys"], q["ablation_per_token_keys"]
    assert q["bits"] == bits
    # ordinary channels: per-token scales are set by the x50 channels
    assert kivi["key_rel_err_ordinary_channels"] * 5 < tok["key_rel_err_ordinary_channels"]
    # per channel, every channel is coded at its own scale: the same relative error
    assert kivi["key_rel_err_outlier_channels"] < 1.5 * kivi["key_rel_err_ordinary_channels"]
    assert kivi["rel_l2"] < tok["rel_l2"] and kivi["cosine"] > tok["cosine"]


def test_committed_report_covers_the_workloads():
    rep = json.load(open(REPORT))
    assert set(rep["workloads"]) == {"tiny", "llama8b_32k", "llama8b_128k_2bit",
                                     "llama8b_128k_4bit", "llama70b_stream"}
    for name, q in rep["workloads"].items():
        kivi, tok = q["kivi_per_channel_keys"], q["ablation_per_token_keys"]
        assert kivi["key_rel_err_ordinary_channels"] * 5 < tok["key_rel_err_ordinary_channels"]
        if name != "tiny":          # 224 quantized tokens: too few for the outputs to part
            assert kivi["rel_l2"] < tok["rel_l2"], name
