"""The byte counter against the figures the pages print (CPU only)."""
import os

import pytest
import sys

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

from quantized_gemv_kv_amd import roofline, synth


def fig(name):
    path = os.path.join(os.path.dirname(__file__), "golden", "page_figures.txt")
    for line in open(path):
        if line.strip() and not line.startswith("#"):
            parts = [p.strip() for p in line.split("|")]
            if parts[0] == name:
                return parts[1]
    raise KeyError(name)


def test_talker_and_predictor_parameter_counts():
    c = synth.config("talker_cp_aff8")
    per_layer = roofline.params_per_layer(c)
    assert per_layer == 15_728_640
    assert round(per_layer / 1e6, 1) == float(fig("talker_params_per_layer")) / 1e6
    talker = c["n_layer"] * per_layer + c["vocab"] * c["d_model"]
    assert talker == 443_547_648
    assert round(talker / 1e6, 1) == float(fig("talker_params_per_step")) / 1e6
    cp = c["cp_n_layer"] * per_layer + c["cp_vocab"] * c["d_model"]
    assert cp == 80_740_352
    assert round(cp / 1e6, 1) == float(fig("cp_params_per_pass")) / 1e6


def test_kv_per_token_and_gb_per_frame():
    c = dict(synth.config("talker_cp_aff8"), batch=1)
    kv = roofline.kv_bytes_per_position(c)
    assert kv == 114_688 and kv / 1024 == float(fig("kv_bytes_per_token"))
    # ~31 MB of KV "at a typical context": about 270 positions
    assert round(270 * kv / 1e6) == 31
    talker_w = c["n_layer"] * roofline.layer_weight_bytes(c) + roofline.matrix_bytes("aff8", c["vocab"], c["d_model"])
    assert talker_w == 471_269_376
    cp_w = 15 * (c["cp_n_layer"] * roofline.layer_weight_bytes(c) + roofline.matrix_bytes("aff8", c["cp_vocab"], c["d_model"]))
    assert cp_w == 15 * 85_786_624
    assert round(cp_w / 1e9, 2) == float(fig("cp_gb_per_frame"))
    # the page's 0.50 GB for the Talker matches its weights plus the typical-context cache
    assert round((talker_w + 270 * kv) / 1e9, 2) == float(fig("talker_gb_per_frame"))
    assert round((talker_w + 270 * kv + cp_w) / 1e9, 2) == float(fig("frame_gb"))


def test_q4_0_row_and_gpt2_step():
    assert roofline.matrix_bytes("q4_0", 1, 1024) == 576
    c = synth.config("gpt2_medium_q4_0")
    b = roofline.step_bytes(c, 255)
    fixed = b["weights"] + b["vectors"] + b["embedding"]
    assert fixed == 175_882_240
    assert b["kv"] == 98_304 * 256
    mean = roofline.mean_step_bytes(c, 256, 500)
    assert abs(mean / 1e6 - 225.7) < 0.05
    # one GPT-2-Medium layer at position 512 (512 prior positions + the new one)
    c2 = synth.config("gpt2_layer_q4_0")
    layer = roofline.layer_weight_bytes(c2)
    assert layer == 7_077_888
    assert roofline.kv_bytes_per_position(c2) * 513 == 2_097_152 + 4_096


def test_llama_step():
    c = synth.config("llama520m_q8_0")
    b = roofline.step_bytes(c, 299)
    assert b["weights"] == 543_686_656
    assert b["vectors"] == 249_856
    assert abs(roofline.mean_step_bytes(c, 300, 600) / 1e6 - 617.7) < 0.1


def test_parity_metric_reproduces_page_rows():
    # rel = max_abs / max|ref|, as in the journal's staged parity table (printed to 2 digits)
    import numpy as np
    from parity import rel_err
    for row in ("parity_row_layer0", "parity_row_layer14", "parity_row_logits_cond", "parity_row_cond_emb"):
        max_abs, max_ref, rel = (float(t) for t in fig(row).split())
        ref = np.array([0.3 * max_ref, -max_ref, 0.5 * max_ref])
        got = ref + np.array([0.0, 0.2 * max_abs, -max_abs])
        assert abs(rel_err(got, ref) - rel) / rel < 0.06, row


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0", "aff8", "q5_0", "aff4_g64", "aff4_g32"])
def test_matrix_bytes_agree_with_the_oracle(orc, fmt):
    for N, K in [(1, 1024), (3072, 1024), (1024, 4096), (7, 192)]:
        if orc.matrix_bytes(fmt, N, K):
            assert roofline.matrix_bytes(fmt, N, K) == orc.matrix_bytes(fmt, N, K)
