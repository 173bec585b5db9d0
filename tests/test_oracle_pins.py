"""The oracle against what the pages and the mathematics fix (CPU only)."""
import math

import numpy as np
import pytest

import oracle
from oracle import kv_math
from oracle_pins import ATTENTION_PINS, golden


@pytest.mark.parametrize("pin", ATTENTION_PINS, ids=lambda p: p.__name__)
def test_attention_pin(pin):
    pin(oracle)


def test_group_size_rejects_irregular_groupings():
    with pytest.raises(ValueError):
        oracle.group_size(6, 4)
    with pytest.raises(ValueError):
        oracle.group_size(8, 0)
    assert oracle.group_size(32, 8) == 4


def test_raw_cache_mib():
    f = golden("kv_cache_figures.json")["raw_cache_mib"]
    for kv, mib in f["by_kv_heads"].items():
        got = kv_math.kv_cache_bytes(f["layers"], f["tokens"], int(kv), f["head_dim"], f["bytes_per_elem"])
        assert got == mib * 2 ** 20
    # a ragged batch sums the actual lengths
    assert kv_math.kv_cache_bytes(2, [3, 5], 1, 4, 2) == kv_math.kv_cache_bytes(2, 8, 1, 4, 2)


def test_qwen3_8b_per_token_and_request():
    f = golden("kv_cache_figures.json")["qwen3_8b_per_token"]
    per = kv_math.kv_bytes_per_token(f["layers"], f["kv_heads"], f["head_dim"], f["bytes_per_elem"])
    assert per == f["bytes_per_token"] and per == f["kib_per_token"] * 1024
    gib = per * f["request_tokens"] / 2 ** 30
    # printed to two decimals (1.125 shown as 1.13)
    assert abs(gib - f["gib_per_request_printed"]) <= 0.005 + 1e-12


def test_qwen3_8b_dial():
    f = golden("kv_cache_figures.json")["qwen3_8b_dial"]
    for kv, kib in f["kib_per_token_by_kv_heads"].items():
        assert kv_math.kv_bytes_per_token(f["layers"], int(kv), f["head_dim"], f["bytes_per_elem"]) == kib * 1024
    flops = kv_math.decode_attention_flops(f["layers"], f["q_heads"], f["head_dim"], f["context_tokens"])
    assert round(flops / 1e9, 2) == f["gflop_per_sequence_step_printed"]
    for kv, ratio in f["flops_per_byte_by_kv_heads"].items():
        per_tok_bytes = kv_math.kv_bytes_per_token(f["layers"], int(kv), f["head_dim"], f["bytes_per_elem"])
        per_tok_flops = kv_math.decode_attention_flops(f["layers"], f["q_heads"], f["head_dim"], 1)
        assert per_tok_flops / per_tok_bytes == ratio


def test_per_token_table():
    f = golden("kv_cache_figures.json")["per_token_table_kb"]
    got = {}
    for name, m in f["models"].items():
        got[name] = kv_math.kv_bytes_per_token(m["layers"], m["kv_heads"], m["head_dim"], f["bytes_per_elem"])
        assert got[name] == m["kb"] * 1024, name
    assert got["LLaMA-2-7B"] == f["ratio_mha_over_gqa"] * got["LLaMA-3-8B"]


def test_concurrency_exercise():
    f = golden("kv_cache_figures.json")["concurrency_exercise"]
    gib = 2 ** 30
    for name in ("LLaMA-3-8B", "LLaMA-2-7B"):
        m = f[name]
        per = kv_math.kv_bytes_per_token(m["layers"], m["kv_heads"], m["head_dim"], 2)
        n = kv_math.max_concurrent_requests(f["gpu_gib"] * gib, m["weights_gib"] * gib,
                                            f["reserve_gib"] * gib, per, f["tokens_per_request"])
        assert n == m["requests"], name


def test_causal_prefill_flops_closed_form():
    # sum over rows i of 4*d*(i+1), checked by direct summation
    B, Hq, N, d = 2, 3, 37, 16
    direct = sum(4 * d * (i + 1) for i in range(N)) * B * Hq
    assert kv_math.causal_prefill_flops(B, Hq, N, d) == direct
    assert kv_math.causal_prefill_flops(2, 32, 4096, 128) == 274945015808
