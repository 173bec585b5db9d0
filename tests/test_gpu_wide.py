"""GPU decode over wide key=value rows (the absorbed-MLA shape, bf16 MFMA
kernel through the C ABI) against the float64 oracle."""
import zlib

import numpy as np
import pytest
import torch

import gqa_inputs as gi
import grouped_query_attention_gqa_amd as gqa
import oracle
from gpu_util import TOL, dev, max_err, need_gpu, say

pytestmark = pytest.mark.gpu

DK, DV = 576, 512


def run_wide(inp, split_tokens=0, scale=None):
    scale = inp.cfg.scale if scale is None else scale
    out = gqa.gqa_decode_wide(dev(inp.q, "bf16"), dev(inp.kv_cache, "bf16"),
                              torch.from_numpy(inp.seq_lens).cuda(), DV, scale=scale,
                              split_tokens=split_tokens)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def ref_wide(inp, scale=None, batch=None):
    scale = inp.cfg.scale if scale is None else scale
    sl = slice(None) if batch is None else slice(batch, batch + 1)
    return oracle.decode_wide(gi.to_f64(inp.q[sl], "bf16"), gi.to_f64(inp.kv_cache[sl], "bf16"),
                              inp.seq_lens[sl], DV, scale)


SMALL = [
    # B, Hq, Hkv, lens, cap
    (2, 128, 1, (100, 37), 128),        # the MLA head count, ragged tails
    (1, 64, 1, (1,), 8),                # a single token
    (3, 128, 2, (300, 0, 65), 320),     # two KV heads (g = 64) and an empty sequence
    (1, 40, 1, (77,), 96),              # g = 40: a partly filled head block
    (2, 192, 1, (200, 150), 256),       # g = 192: three head blocks
    (4, 16, 4, (33, 64, 95, 2), 96),    # g = 4: mostly idle heads in the block
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}-{}on{}-T{}".format(c[0], c[1], c[2], max(c[3])))
def test_small_wide_parity(case):
    need_gpu()
    B, Hq, Hkv, lens, cap = case
    inp = gi.small_wide(B, Hq, Hkv, DK, DV, list(lens), cap, seed=zlib.crc32(repr(case).encode()) % 100000)
    say("wide small", case)
    got = run_wide(inp)
    err = max_err(got, ref_wide(inp))
    say("max err", err)
    assert err <= TOL["bf16"]
    for b, t in enumerate(lens):
        if t == 0:
            assert np.all(got[b] == 0)


@pytest.mark.parametrize("split", [32, 64, 96])
def test_forced_ranges_merge(split):
    """Several token ranges per sequence go through the partials and the
    log-sum-exp merge; each result matches the oracle and the one-range run."""
    need_gpu()
    inp = gi.small_wide(3, 128, 1, DK, DV, [250, 31, 129], 256, seed=611)
    say("wide split", split)
    whole = run_wide(inp, split_tokens=256)
    got = run_wide(inp, split_tokens=split)
    ref = ref_wide(inp)
    e1, e2 = max_err(got, ref), max_err(whole, ref)
    say("max err split", e1, "one range", e2)
    assert e1 <= TOL["bf16"] and e2 <= TOL["bf16"]


def test_late_large_score_second_pass():
    """A token well after the first tile whose score exceeds every earlier
    one by far (about 2^84 in weight for head 0, beyond the kernel's 2^32
    slack): the kernel must recompute the range against the true maximum.
    Checked against the oracle, whose output is then dominated by that
    token."""
    need_gpu()
    inp = gi.small_wide(1, 64, 1, DK, DV, [200], 224, seed=617)
    q = gi.bf16_bits_to_f32(inp.q[0, 0])
    row = np.sign(q) * 2.0                      # aligned with head 0's query
    inp.kv_cache[0, 0, 150] = gi.f32_to_bf16_bits(row.astype(np.float32))
    got = run_wide(inp)
    ref = ref_wide(inp)
    err = max_err(got, ref)
    say("late max err", err)
    assert err <= TOL["bf16"]
    assert np.max(np.abs(ref[0, 0] - gi.to_f64(inp.kv_cache[0, 0, 150, :DV], "bf16"))) < 1e-3


def test_group_mapping_wide():
    """Query heads 0..63 read KV head 0 and 64..127 KV head 1: identical
    queries in two groups over different rows give different outputs, and
    within a group identical queries give identical outputs."""
    need_gpu()
    inp = gi.small_wide(1, 128, 2, DK, DV, [90], 96, seed=619)
    inp.q[0, 1] = inp.q[0, 0]
    inp.q[0, 64] = inp.q[0, 0]
    got = run_wide(inp)
    assert np.array_equal(got[0, 0], got[0, 1])
    assert not np.allclose(got[0, 0], got[0, 64])
    assert max_err(got, ref_wide(inp)) <= TOL["bf16"]


_FULL = {}


@pytest.mark.parametrize("part", range(4))
def test_mla_decode_full(part):
    """Every output row of the mla-decode workload (B=64, Hq=128, Hkv=1,
    576/512, T=4096) in the bench's launch configuration, a quarter of the
    batch per test, one sequence per oracle call."""
    need_gpu()
    cfg = gi.WIDE_CONFIGS["mla-decode"]
    if "w" not in _FULL:
        inp = gi.make_wide(cfg)
        say("mla-decode", gi.describe(cfg))
        _FULL["w"] = (inp, run_wide(inp))
    inp, got = _FULL["w"]
    worst = 0.0
    for b in range(16 * part, 16 * part + 16):
        worst = max(worst, max_err(got[b:b + 1], ref_wide(inp, batch=b)))
    say("mla-decode part", part, "max err", worst)
    assert worst <= TOL["bf16"]
