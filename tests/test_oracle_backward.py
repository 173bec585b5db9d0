"""The prefill-gradient oracle against its pins, and planted mistakes (CPU only)."""
import os
import types

import numpy as np
import pytest

import oracle
from oracle import backward as backward_mod
from backward_pins import BACKWARD_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "backward.py")


@pytest.mark.parametrize("pin", BACKWARD_PINS, ids=lambda p: p.__name__)
def test_backward_pin(pin):
    pin(backward_mod)


def test_rejects_bad_grouping():
    with pytest.raises(ValueError):
        oracle.prefill_causal_backward(np.zeros((1, 3, 2, 2)), np.zeros((1, 2, 2, 2)),
                                       np.zeros((1, 2, 2, 2)), np.zeros((1, 3, 2, 2)), 1.0)


def test_empty_prompt():
    z = np.zeros((1, 2, 0, 4))
    dq, dk, dv = oracle.prefill_causal_backward(z, z[:, :1], z[:, :1], z, 1.0)
    assert dq.shape == (1, 2, 0, 4) and dk.shape == (1, 1, 0, 4) and dv.shape == (1, 1, 0, 4)


MUTANTS = {
    "no_group_sum": ("out = x.reshape((hq // g, g) + x.shape[1:]).sum(axis=1)",
                     "out = x.reshape((hq // g, g) + x.shape[1:])[:, 0]"),
    "strided_grouping": ("out = x.reshape((hq // g, g) + x.shape[1:]).sum(axis=1)",
                         "out = x.reshape((g, hq // g) + x.shape[1:]).sum(axis=0)"),
    "no_softmax_correction": ("ds = p * (dp - np.sum(p * dp, axis=-1, keepdims=True))", "ds = p * dp"),
    "flipped_sign": ("ds = p * (dp - np.sum(p * dp, axis=-1, keepdims=True))",
                     "ds = p * (np.sum(p * dp, axis=-1, keepdims=True) - dp)"),
    "column_correction": ("ds = p * (dp - np.sum(p * dp, axis=-1, keepdims=True))",
                          "ds = p * (dp - np.sum(p * dp, axis=0, keepdims=True))"),
    "dq_unscaled": ("dq_h = scale * (ds @ k_h)", "dq_h = ds @ k_h"),
    "dq_transposed": ("dq_h = scale * (ds @ k_h)", "dq_h = scale * (ds.T @ k_h)"),
    "dk_from_keys": ("dk_h = scale * (ds.T @ q_h)", "dk_h = scale * (ds.T @ k_h)"),
    "dv_untransposed": ("dv_h = p.T @ do_h", "dv_h = p @ do_h"),
    "no_causal_mask": ("s = _causal_scores(q_h, k_h, np.arange(n), scale)", "s = scale * (q_h @ k_h.T)"),
    "dp_from_keys": ("dp = do_h @ v_h.T", "dp = do_h @ k_h.T"),
}


def _load(name):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        text = f.read()
    assert old in text, name
    text = text.replace(old, new).replace("from .attention import", "from oracle.attention import")
    mod = types.ModuleType(f"backward_mutant_{name}")
    exec(compile(text, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_backward_mutant(name):
    mod = _load(name)
    caught = []
    for pin in BACKWARD_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except Exception as e:
            caught.append(f"{pin.__name__}: {type(e).__name__}")
    assert caught, f"no pin caught mutant {name}"
