"""The FP8 cache oracle against its pins, and planted mistakes (CPU only)."""
import os
import types

import numpy as np
import pytest

from oracle import fp8 as fp8_mod
from fp8_pins import FP8_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "fp8.py")


@pytest.mark.parametrize("pin", FP8_PINS, ids=lambda p: p.__name__)
def test_fp8_pin(pin):
    pin(fp8_mod)


MUTANTS = {
    "bias_8": ("(8.0 + m) * 2.0 ** (e - 10.0)", "(8.0 + m) * 2.0 ** (e - 11.0)"),
    "subnormal_as_normal": ("np.where(e == 0, m * 2.0 ** -9,", "np.where(e < 0, m * 2.0 ** -9,"),
    "nan_code_finite": ("mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)", "mag = mag"),
    "sign_ignored": ("sign = np.where(c & 0x80, -1.0, 1.0)", "sign = 1.0"),
    "scale_per_token_axis": ("[None, :, None, None]", "[None, None, :, None] if False else np.asarray(scales, dtype=np.float64).mean()"),
    "v_scale_for_k": ("dequantize(k_codes, k_scale)", "dequantize(k_codes, v_scale)"),
    "mantissa_dropped": ("(8.0 + m) * 2.0 ** (e - 10.0)", "8.0 * 2.0 ** (e - 10.0)"),
}


def _load(name):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        text = f.read()
    assert old in text, name
    text = text.replace(old, new).replace("from .attention import decode", "from oracle.attention import decode")
    mod = types.ModuleType(f"fp8_mutant_{name}")
    exec(compile(text, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_fp8_mutant(name):
    mod = _load(name)
    caught = []
    for pin in FP8_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except Exception as e:
            caught.append(f"{pin.__name__}: {type(e).__name__}")
    assert caught, f"no pin caught mutant {name}"
