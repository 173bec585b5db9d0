"""The paged-cache oracle against its pins, and planted mistakes (CPU only)."""
import os
import types

import numpy as np
import pytest

import oracle
from oracle import paged as paged_mod
from paged_pins import PAGED_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "paged.py")


@pytest.mark.parametrize("pin", PAGED_PINS, ids=lambda p: p.__name__)
def test_paged_pin(pin):
    pin(paged_mod)


def test_rejects_page_outside_pool():
    pages = np.zeros((3, 1, 2, 4))
    with pytest.raises(ValueError):
        oracle.gather_pages(pages, np.array([[0, 5]], dtype=np.int32), np.array([4]), 2)


MUTANTS = {
    "next_table_entry": ("pid = int(table[b, i])", "pid = int(table[b, min(i + 1, max_pages - 1)])"),
    "head_zero_for_all": ("out[b, :, i * page_size:i * page_size + n] = pages[pid, :, :n]",
                          "out[b, :, i * page_size:i * page_size + n] = pages[pid, :1, :n]"),
    "rows_shifted": ("out[b, :, i * page_size:i * page_size + n] = pages[pid, :, :n]",
                     "out[b, :, i * page_size:i * page_size + n] = np.roll(pages[pid], 1, axis=1)[:, :n]"),
    "value_from_key_pages": ("v = gather_pages(np.asarray(v_pages", "v = gather_pages(np.asarray(k_pages"),
    "identity_table": ("pid = int(table[b, i])", "pid = (b * max_pages + i) % pages.shape[0]"),
}


def _load(name):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        text = f.read()
    assert old in text, name
    text = text.replace(old, new).replace("from .attention import decode", "from oracle.attention import decode")
    mod = types.ModuleType(f"paged_mutant_{name}")
    exec(compile(text, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_paged_mutant(name):
    mod = _load(name)
    caught = []
    for pin in PAGED_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except Exception as e:
            caught.append(f"{pin.__name__}: {type(e).__name__}")
    assert caught, f"no pin caught mutant {name}"
