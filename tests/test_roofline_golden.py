"""The roofline arithmetic against the numbers the pages print (tests/golden)."""
import json
import os

import pytest

import synth
from memory_bound_transformer_persistent_amd import roofline as R

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_arithmetic.json")))


@pytest.mark.parametrize("case", GOLD["bandwidth_bound"], ids=["h200", "mi300x"])
def test_bandwidth_bound_reproduces_pages(case):
    w = case["params"] * case["bytes_per_param"]
    tps = R.bound_tokens_per_s(case["bw_bytes_per_s"], w, case["kv_bytes"], case["beta"])
    step = case["printed_rounding"]
    assert round(tps / step) * step == case["printed_tokens_per_s"]


def test_launch_overhead_model_reproduces_pages():
    c = GOLD["launch_overhead"]
    us, cap = R.launch_overhead(c["launch_us"], c["kernels_per_layer"], c["layers"])
    assert us == c["printed_us_per_token"]
    assert round(cap / c["printed_rounding"]) * c["printed_rounding"] == c["printed_tokens_per_s"]


def test_token_budget_and_long_generation_arithmetic():
    b = GOLD["token_budget"]
    us = 1e6 / b["tokens_per_s"]
    assert int(us) == b["printed_us_per_token"]
    assert round(us / b["layers"], 1) == b["printed_us_per_layer"]
    g = GOLD["long_generation"]
    assert round(g["tokens"] / g["slow_tokens_per_s"] / 60) == g["printed_slow_minutes"]
    assert g["tokens"] / g["fast_tokens_per_s"] < g["printed_fast_seconds_below"]


def test_dense2b_step_bytes():
    s = synth.shape_for("dense2b")
    # 25 x (3*2560^2 + 2560^2 + 3*6912*2560 + 2*2560) + 2560 + 65536*2560 fp16 values
    assert R.weight_bytes(s) == 2 * (25 * (4 * 2560 * 2560 + 3 * 6912 * 2560 + 2 * 2560)
                                     + 2560 + 65536 * 2560)
    sb = R.step_bytes(s, pos=0)
    assert sb.kv_read == 256_000 and sb.kv_write == 256_000
    # beta = 1 roofline for the 128-prompt + 512-step run lands near 1,818 tok/s
    tps = R.roofline_tokens_per_s(s, first_pos=128, n_steps=512)
    assert 1800 < tps < 1830
    # bytes grow by exactly one KV row per position
    assert R.step_bytes(s, 10).total - R.step_bytes(s, 9).total == 256_000


def test_batch_reads_weights_once():
    s = synth.shape_for("dense2b")
    b1, b8 = R.step_bytes(s, 300, 1), R.step_bytes(s, 300, 8)
    assert b8.weights == b1.weights and b8.kv_read == 8 * b1.kv_read
