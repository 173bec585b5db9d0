"""The wide-row (absorbed-MLA) decode oracle against its pins, and planted
mistakes (CPU only)."""
import os
import types

import numpy as np
import pytest

import oracle
from oracle import wide as wide_mod
from wide_pins import WIDE_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "wide.py")


@pytest.mark.parametrize("pin", WIDE_PINS, ids=lambda p: p.__name__)
def test_wide_pin(pin):
    pin(wide_mod)


def test_rejects_bad_value_width():
    with pytest.raises(ValueError):
        oracle.decode_wide(np.zeros((1, 2, 4)), np.zeros((1, 1, 3, 4)), np.array([3]), 5, 1.0)


MUTANTS = {
    "value_from_trailing_columns": ("softmax_average(s, rows[..., :d_v])", "softmax_average(s, rows[..., -d_v:])"),
    "scores_without_rotary": ("s = scale * np.matmul(rows, q[b][:, :, None])[..., 0]",
                              "s = scale * np.matmul(rows[..., :d_v], q[b][:, :d_v, None])[..., 0]"),
    "strided_heads": ("rows = expand_kv_heads(_as_f64(kv_cache[b, :, :T]), g, axis=0)",
                      "rows = np.tile(_as_f64(kv_cache[b, :, :T]), (g, 1, 1))"),
    "scale_dropped": ("s = scale * np.matmul(rows, q[b][:, :, None])[..., 0]",
                      "s = np.matmul(rows, q[b][:, :, None])[..., 0]"),
    "one_token_short": ("rows = expand_kv_heads(_as_f64(kv_cache[b, :, :T]), g, axis=0)",
                        "rows = expand_kv_heads(_as_f64(kv_cache[b, :, :max(T - 1, 1)]), g, axis=0)"),
}


def _load(name):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        text = f.read()
    assert old in text, name
    text = text.replace(old, new).replace("from .attention import", "from oracle.attention import")
    mod = types.ModuleType(f"wide_mutant_{name}")
    exec(compile(text, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_wide_mutant(name):
    mod = _load(name)
    caught = []
    for pin in WIDE_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except Exception as e:
            caught.append(f"{pin.__name__}: {type(e).__name__}")
    assert caught, f"no pin caught mutant {name}"
