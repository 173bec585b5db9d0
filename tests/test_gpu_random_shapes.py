"""Seeded random shapes through the C ABI against the float64 oracle: decode
(bf16 and fp32 caches, automatic and caller-fixed ranges, one call and the
two stages), paged and E4M3 caches, wide rows, causal prefill and its
backward.

The shapes come from one generator with a fixed seed, so every case is
reproducible from its id.  They reach what the hand-picked cases do not:
group sizes that are not powers of two (3, 5, 7, 12, 20, 31, 33, 40), one to
four KV heads, capacities that are no multiple of any tile, lengths of zero
and at capacity in the same batch, and range sizes down to one 32-token
quantum.  Tolerances are the other GPU tests': max |gpu - oracle| <= 2e-2 for
bf16 and 1e-5 for fp32 decode, the relative gradient bound for the
backward; prefill row 0 must equal V[0] exactly."""
import numpy as np
import pytest

import gqa_inputs as gi
import oracle
from gpu_util import TOL, max_err, need_gpu, say
from test_gpu_backward import TOL_REL, oracle_grads, rel_err, run_backward
from test_gpu_decode import oracle_full, run_decode
from test_gpu_fp8 import fp8_oracle, run_fp8
from test_gpu_paged import paged_oracle, run_contiguous, run_paged
from test_gpu_prefill import run_prefill
from test_gpu_wide import DK, DV, ref_wide, run_wide

pytestmark = pytest.mark.gpu

_rng = np.random.default_rng(0x6A5)


def _decode_cases(n):
    cases = []
    for i in range(n):
        dtype = "f32" if i % 6 == 5 else "bf16"
        hkv = int(_rng.choice([1, 2, 3, 4]))
        g = int(_rng.choice([1, 2, 3, 4, 5, 7, 8, 12, 16, 20, 31, 32, 33, 40]))
        d = int(_rng.choice([64, 128]))
        b = int(_rng.integers(1, 6))
        tcap = int(_rng.integers(1, 2500))
        lens = _rng.integers(0, tcap + 1, size=b)
        if b > 1:
            lens[int(_rng.integers(0, b))] = tcap          # one sequence at capacity
        if b > 2 and i % 3 == 0:
            lens[int(_rng.integers(0, b))] = 0             # and, every third case, an empty one
        split = int(_rng.choice([0, 0, 32, 64, 96, 256, 1024]))
        stages = bool(i % 2)
        cases.append((dtype, b, g * hkv, hkv, d, tcap, tuple(int(t) for t in lens), split, stages))
    return cases


def _prefill_cases(n, max_n, max_hq):
    cases = []
    while len(cases) < n:
        b = int(_rng.integers(1, 3))
        hkv = int(_rng.choice([1, 2, 3]))
        g = int(_rng.choice([1, 2, 3, 4, 5, 6, 8, 12]))
        if g * hkv > max_hq:
            continue
        seq = int(_rng.integers(1, max_n + 1))
        cases.append((b, g * hkv, hkv, seq, (64, 128)[len(cases) % 2]))
    return cases


def _cache_cases(n, paged):
    cases = []
    for i in range(n):
        hkv = int(_rng.choice([1, 2, 3]))
        g = int(_rng.choice([1, 3, 4, 6, 16, 24, 32, 40, 71]))
        d = int(_rng.choice([64, 128]))
        b = int(_rng.integers(1, 5))
        if paged:
            extra = int(_rng.choice([1, 2, 4, 8, 16, 32, 64, 256]))   # page size
            tcap = extra * int(_rng.integers(1, max(2, 2048 // extra)))
        else:
            extra = int(_rng.choice([0, 0, 32, 64, 160, 512]))       # range size
            tcap = int(_rng.integers(1, 2048))
        lens = _rng.integers(0, tcap + 1, size=b)
        lens[int(_rng.integers(0, b))] = tcap
        cases.append((b, g * hkv, hkv, d, tcap, tuple(int(t) for t in lens), extra))
    return cases


def _wide_cases(n):
    cases = []
    for i in range(n):
        hkv = int(_rng.choice([1, 2]))
        g = int(_rng.choice([4, 16, 40, 64, 100, 128, 192]))
        b = int(_rng.integers(1, 5))
        cap = int(_rng.integers(1, 600))
        lens = _rng.integers(0, cap + 1, size=b)
        lens[int(_rng.integers(0, b))] = cap
        split = int(_rng.choice([0, 0, 32, 64, 160]))
        cases.append((b, g * hkv, hkv, cap, tuple(int(t) for t in lens), split))
    return cases


DECODE = _decode_cases(24)
PREFILL = _prefill_cases(12, 600, 36)
BACKWARD = _prefill_cases(6, 400, 16)
PAGED = _cache_cases(8, paged=True)
FP8 = _cache_cases(8, paged=False)
WIDE = _wide_cases(6)


def _many_block_cases(n):
    """head_dim 64 with groups of 33 to 96 heads: units of three to five
    16-head blocks (and a second unit past 80 heads)."""
    cases = []
    for i in range(n):
        hkv = int(_rng.choice([1, 2]))
        g = int(_rng.integers(33, 97))
        b = int(_rng.integers(1, 5))
        tcap = int(_rng.integers(1, 3000))
        lens = _rng.integers(0, tcap + 1, size=b)
        lens[int(_rng.integers(0, b))] = tcap
        split = int(_rng.choice([0, 0, 64, 256]))
        cases.append(("fp8" if i % 4 == 3 else "bf16", b, g * hkv, hkv, tcap, tuple(int(t) for t in lens), split,
                      bool(i % 2)))
    return cases


MANY_BLOCKS = _many_block_cases(8)


def _cache_id(c):
    return "B{}-{}on{}-d{}-T{}-{}".format(*c[:5], c[6])


def _decode_id(c):
    dtype, b, hq, hkv, d, tcap, lens, split, stages = c
    return f"{dtype}-B{b}-{hq}on{hkv}-d{d}-T{tcap}-split{split}-{'stages' if stages else 'call'}"


@pytest.mark.parametrize("case", DECODE, ids=_decode_id)
def test_random_decode_shapes(case):
    need_gpu()
    dtype, b, hq, hkv, d, tcap, lens, split, stages = case
    inp = gi.small_decode(dtype, b, hq, hkv, d, list(lens), tcap, seed=sum(lens) % 9973 + hq)
    say("random decode", _decode_id(case), "lens", list(lens))
    got = run_decode(inp, split_tokens=split, stages=stages)
    err = max_err(got, oracle_full(inp))
    say("max err", err)
    assert err <= TOL[dtype]
    for i, t in enumerate(lens):
        if t == 0:
            assert np.all(got[i] == 0.0)


@pytest.mark.parametrize("case", PREFILL, ids=lambda c: "B{}-{}on{}-N{}-d{}".format(*c))
def test_random_prefill_shapes(case):
    need_gpu()
    B, Hq, Hkv, N, d = case
    p = gi.small_prefill(B, Hq, Hkv, N, d, seed=N * 31 + Hq)
    say("random prefill", case)
    out, lse = run_prefill(p)
    ref, ref_lse = oracle.prefill_causal(gi.to_f64(p.q, "bf16"), gi.to_f64(p.k, "bf16"),
                                         gi.to_f64(p.v, "bf16"), p.cfg.scale, return_lse=True)
    err, lerr = max_err(out, ref), max_err(lse, ref_lse)
    say("max err", err, "lse err", lerr)
    assert err <= TOL["bf16"] and lerr <= TOL["bf16"]
    g = Hq // Hkv
    for bb in range(B):
        for h in range(Hq):
            assert np.array_equal(out[bb, h, 0], gi.bf16_bits_to_f32(p.v[bb, h // g, 0]))


@pytest.mark.parametrize("case", BACKWARD, ids=lambda c: "B{}-{}on{}-N{}-d{}".format(*c))
def test_random_backward_shapes(case):
    need_gpu()
    B, Hq, Hkv, N, d = case
    p = gi.small_prefill(B, Hq, Hkv, N, d, seed=N * 37 + Hq)
    do = gi.make_dout(p.cfg)
    say("random backward", case)
    errs = [rel_err(a, r) for a, r in zip(run_backward(p, do), oracle_grads(p, do))]
    say("rel err dq dk dv", errs)
    assert max(errs) <= TOL_REL


@pytest.mark.parametrize("case", PAGED, ids=_cache_id)
def test_random_paged_shapes(case):
    """The paged result also equals the contiguous cache's bit for bit."""
    need_gpu()
    B, Hq, Hkv, d, T, lens, ps = case
    inp = gi.small_decode("bf16", B, Hq, Hkv, d, list(lens), T, seed=sum(lens) % 9973 + Hq)
    pg = gi.make_paged(inp, page_size=ps, seed=ps + 3)
    say("random paged", _cache_id(case), "lens", list(lens), "pool pages", pg.k_pages.shape[0])
    got = run_paged(pg)
    err = max_err(got, paged_oracle(pg))
    say("max err", err)
    assert err <= TOL["bf16"]
    assert np.array_equal(got, run_contiguous(inp))


@pytest.mark.parametrize("case", FP8, ids=_cache_id)
def test_random_fp8_shapes(case):
    need_gpu()
    B, Hq, Hkv, d, T, lens, split = case
    inp = gi.small_decode("bf16", B, Hq, Hkv, d, list(lens), T, seed=sum(lens) % 9973 + 2 * Hq)
    fp = gi.make_fp8(inp)
    say("random fp8", _cache_id(case), "lens", list(lens))
    err = max_err(run_fp8(fp, split), fp8_oracle(fp))
    say("max err", err)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("case", WIDE, ids=lambda c: "B{}-{}on{}-T{}-split{}".format(c[0], c[1], c[2], c[3], c[5]))
def test_random_wide_shapes(case):
    need_gpu()
    B, Hq, Hkv, cap, lens, split = case
    inp = gi.small_wide(B, Hq, Hkv, DK, DV, list(lens), cap, seed=sum(lens) % 9973 + Hq)
    say("random wide", case)
    got = run_wide(inp, split)
    err = max_err(got, ref_wide(inp))
    say("max err", err)
    assert err <= TOL["bf16"]
    for b, t in enumerate(lens):
        if t == 0:
            assert np.all(got[b] == 0)


@pytest.mark.parametrize("case", MANY_BLOCKS,
                         ids=lambda c: "{}-B{}-{}on{}-d64-T{}-split{}-{}".format(*c[:5], c[6], "stages" if c[7] else "call"))
def test_random_many_block_units(case):
    need_gpu()
    kind, B, Hq, Hkv, T, lens, split, stages = case
    inp = gi.small_decode("bf16", B, Hq, Hkv, 64, list(lens), T, seed=sum(lens) % 9973 + 3 * Hq)
    say("random many-block", case)
    if kind == "fp8":
        fp = gi.make_fp8(inp)
        err = max_err(run_fp8(fp, split), fp8_oracle(fp))
    else:
        err = max_err(run_decode(inp, split_tokens=split, stages=stages), oracle_full(inp))
    say("max err", err)
    assert err <= TOL["bf16"]
