"""Plant plausible mistakes in a copy of the oracle and check the pins catch
each one.  The mutants live only in memory, on the CPU."""
import importlib.util
import os
import types

import pytest

from oracle_pins import ATTENTION_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "attention.py")

MUTANTS = {
    "tile_instead_of_repeat": ("return np.repeat(x, g, axis=axis)",
                               "reps = [1] * np.ndim(x); reps[axis] = g; return np.tile(x, reps)"),
    "mapping_modulo": ("return h // group_size(num_q_heads, num_kv_heads)",
                       "return h % num_kv_heads"),
    "decode_drops_scale": ("s = scale * np.matmul(k_exp", "s = np.matmul(k_exp"),
    "no_max_subtraction": ("w = np.exp(scores - m)", "w = np.exp(scores)"),
    "no_normalisation": ("return num / den[..., None], m[..., 0] + np.log(den)",
                         "return num, m[..., 0] + np.log(den)"),
    "lse_without_max": ("m[..., 0] + np.log(den)", "np.log(den)"),
    "causal_mask_flipped": ("np.where(j <= np.asarray(rows)[:, None], s, -np.inf)",
                            "np.where(j >= np.asarray(rows)[:, None], s, -np.inf)"),
    "causal_mask_strict": ("np.where(j <= np.asarray(rows)[:, None], s, -np.inf)",
                           "np.where(j < np.asarray(rows)[:, None] + (np.asarray(rows)[:, None] == 0), s, -np.inf)"),
    "decode_drops_last_token": ("k_exp = expand_kv_heads(_as_f64(k_cache[b, :, :T])",
                                "k_exp = expand_kv_heads(_as_f64(k_cache[b, :, :max(T - 1, 1)])"),
    "value_from_key": ("v_exp = expand_kv_heads(_as_f64(v[b]), g, axis=0)",
                       "v_exp = expand_kv_heads(_as_f64(k[b]), g, axis=0)"),
    "prefill_scale_squared": ("s = scale * (q_rows @ k.T)", "s = scale * scale * (q_rows @ k.T)"),
    "divisibility_unchecked": ("num_q_heads % num_kv_heads != 0", "False"),
}


def _load_mutant(name):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) >= 1, f"mutation site for {name} not found"
    text = text.replace(old, new)
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(text, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    mod = _load_mutant(name)
    caught = []
    for pin in ATTENTION_PINS:
        try:
            with __import__("numpy").errstate(all="ignore"):
                pin(mod)
        except Exception as e:  # AssertionError, or the mutant crashing
            caught.append(f"{pin.__name__}: {type(e).__name__}")
    assert caught, f"no pin caught mutant {name}"
