"""Pins for the byte/FLOP accounting against the pages' worked arithmetic
(tests/golden/pages_arithmetic.json, each entry cited) and hand-checked totals."""
import json
import os

from paged_kv_gqa_qwen3_amd import accounting as acc
from paged_kv_gqa_qwen3_amd import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "pages_arithmetic.json")))


def test_lm_head_logits_bytes():
    g = GOLD["lm_head_prefill_logits_bytes"]
    b = g["tokens"] * g["vocab"] * g["elem_bytes"]
    assert round(b / 1e6) == g["printed_MB"]


def test_kv_bytes_per_token():
    g = GOLD["kv_cache_bytes_per_token"]
    b = acc.kv_bytes_per_token(g["layers"], g["kv_heads"], g["head_dim"], g["elem_bytes"])
    assert b == g["printed_MB"] * 2 ** 20


def test_decode_gemv_intensity():
    g = GOLD["decode_gemv_intensity"]
    flops = acc.gemm_flops(1, g["hidden"], g["hidden"])
    nbytes = g["hidden"] * g["hidden"] * 2
    assert round(flops / 1e6) == g["printed_MFLOP"]
    assert round(nbytes / 1e6) == g["printed_MB"]
    assert flops / nbytes == g["printed_flop_per_byte"]


def test_prefill_projection_flops():
    g = GOLD["prefill_projection_flops"]
    # 2 x 35200 x 8192^2 = 4.7245e12; the page prints "about 4.73", so the check
    # allows the page's last printed digit.
    assert abs(acc.gemm_flops(g["m"], g["n"], g["k"]) / 1e12 - g["printed_TFLOP"]) < 0.01


def test_qwen3_4b_shape_constants():
    g = GOLD["qwen3_4b_shape"]
    s = synth.QWEN3_4B
    assert (s.num_layers, s.hidden, s.num_q_heads, s.num_kv_heads, s.vocab) == \
        (g["layers"], g["hidden"], g["q_heads"], g["kv_heads"], g["vocab"])


def test_attention_call_count():
    g = GOLD["attention_call_count"]
    assert g["requests"] * g["steps"] * g["layers"] == g["printed"]


def test_qwen3_4b_step_bytes():
    s = synth.QWEN3_4B
    # per layer: QKV 6144x2560, O 2560x4096, gate+up 2x9728x2560, down 2560x9728 (bf16)
    per_layer = (6144 * 2560 + 2560 * 4096 + 2 * 9728 * 2560 + 2560 * 9728) * 2
    assert per_layer == 201_850_880
    assert acc.linear_weight_bytes(s) == 36 * per_layer == 7_266_631_680
    assert acc.lm_head_bytes(s) == 777_912_320
    assert acc.norm_bytes(s) == 392_192
    assert acc.kv_bytes_per_token(36, 8, 128) == 147_456
    assert acc.step_bytes(s, [513]) == (8_044_544_000 + 392_192 + 2560 * 2 + 513 * 147_456)


def test_qwen3_8b_untied_bytes():
    s = synth.QWEN3_8B
    assert acc.linear_weight_bytes(s) + acc.lm_head_bytes(s) == 15_136_194_560
