"""GPU causal prefill (bf16 MFMA kernel through the C ABI) against the oracle."""
import zlib

import numpy as np
import pytest
import torch

import gqa_inputs as gi
import grouped_query_attention_gqa_amd as gqa
import oracle
from gpu_util import TOL, dev, max_err, need_gpu, say

pytestmark = pytest.mark.gpu


def run_prefill(p):
    q, k, v = dev(p.q, "bf16"), dev(p.k, "bf16"), dev(p.v, "bf16")
    out, lse = gqa.gqa_prefill_causal(q, k, v, scale=p.cfg.scale, return_lse=True)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


SMALL = [
    # B, Hq, Hkv, N, d
    (1, 8, 2, 300, 128),     # group 4, ragged tail
    (2, 8, 2, 64, 64),
    (1, 4, 4, 130, 128),     # MHA endpoint
    (1, 6, 2, 77, 128),      # group 3: one head per workgroup
    (1, 16, 1, 200, 128),    # MQA, group 16
    (1, 4, 2, 1, 128),       # a single token
    (1, 8, 4, 33, 64),       # group 2
    (1, 8, 4, 1000, 128),    # group 2, 64 positions per q-tile, even q-tile count
    (1, 16, 2, 515, 128),    # group 8 (two head blocks), odd q-tile count
    (2, 4, 1, 640, 64),      # MQA-style group 4, d = 64
    (1, 3, 3, 389, 128),     # MHA, 128 positions per q-tile, split pairs
    (1, 32, 8, 300, 128),    # 8 units: q-tiles of one KV head grouped per XCD (the prefill-4k mapping)
    (2, 16, 8, 200, 64),     # 16 units, d = 64, same mapping
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}-{}on{}-N{}-d{}".format(*c))
def test_small_full_parity(case):
    need_gpu()
    B, Hq, Hkv, N, d = case
    p = gi.small_prefill(B, Hq, Hkv, N, d, seed=zlib.crc32(repr(case).encode()) % 100000)
    say("prefill small", case)
    out, lse = run_prefill(p)
    ref, ref_lse = oracle.prefill_causal(gi.to_f64(p.q, "bf16"), gi.to_f64(p.k, "bf16"),
                                         gi.to_f64(p.v, "bf16"), p.cfg.scale, return_lse=True)
    err, lerr = max_err(out, ref), max_err(lse, ref_lse)
    say("max err", err, "lse err", lerr)
    assert err <= TOL["bf16"] and lerr <= TOL["bf16"]
    # row 0 attends only key 0: exactly V[0]
    g = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            assert np.array_equal(out[b, h, 0], gi.bf16_bits_to_f32(p.v[b, h // g, 0]))


_FULL = {}


@pytest.mark.parametrize("b", [0, 1])
def test_prefill_4k_full(b):
    """Every output row and lse of the prefill-4k workload, one sequence (all
    32 query heads over its 8 KV heads) per test, in the bench's launch."""
    need_gpu()
    cfg = gi.CONFIGS["prefill-4k"]
    if "p" not in _FULL:
        p = gi.make_prefill(cfg)
        say("prefill-4k", gi.describe(cfg))
        _FULL["p"] = (p, *run_prefill(p))
    p, out, lse = _FULL["p"]
    ref, ref_lse = oracle.prefill_causal(gi.to_f64(p.q[b:b + 1], "bf16"), gi.to_f64(p.k[b:b + 1], "bf16"),
                                         gi.to_f64(p.v[b:b + 1], "bf16"), cfg.scale, return_lse=True)
    err, lerr = max_err(out[b:b + 1], ref), max_err(lse[b:b + 1], ref_lse)
    say("prefill-4k sequence", b, "max err", err, "lse err", lerr)
    assert err <= TOL["bf16"] and lerr <= TOL["bf16"]


def test_causality_perturbation_bit_identical():
    need_gpu()
    p = gi.small_prefill(1, 8, 2, 256, 128, seed=31)
    out_a, _ = run_prefill(p)
    i = 100
    p.k[:, :, i + 1:] = gi.f32_to_bf16_bits(gi.bf16_bits_to_f32(p.k[:, :, i + 1:]) * 2.0 + 1.0)
    p.v[:, :, i + 1:] = gi.f32_to_bf16_bits(gi.bf16_bits_to_f32(p.v[:, :, i + 1:]) - 3.0)
    out_b, _ = run_prefill(p)
    assert np.array_equal(out_a[:, :, :i + 1], out_b[:, :, :i + 1])
    assert not np.allclose(out_a[:, :, i + 1:], out_b[:, :, i + 1:])


def test_identical_queries_in_group_identical_rows():
    need_gpu()
    p = gi.small_prefill(1, 4, 1, 96, 128, seed=41)
    p.q[:, 1] = p.q[:, 0]
    out, _ = run_prefill(p)
    assert np.array_equal(out[0, 0], out[0, 1])
    assert not np.allclose(out[0, 0], out[0, 2])


@pytest.mark.parametrize("scale", [0.0, -0.07], ids=["zero", "negative"])
def test_nonpositive_scale(scale):
    need_gpu()
    p = gi.small_prefill(1, 8, 2, 200, 128, seed=53)
    q, k, v = dev(p.q, "bf16"), dev(p.k, "bf16"), dev(p.v, "bf16")
    out, lse = gqa.gqa_prefill_causal(q, k, v, scale=scale, return_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.prefill_causal(gi.to_f64(p.q, "bf16"), gi.to_f64(p.k, "bf16"),
                                         gi.to_f64(p.v, "bf16"), scale, return_lse=True)
    err, lerr = max_err(out.cpu().numpy(), ref), max_err(lse.cpu().numpy(), ref_lse)
    say("scale", scale, "max err", err, "lse err", lerr)
    assert err <= TOL["bf16"] and lerr <= TOL["bf16"]


def test_large_scale_moves_reference_often():
    """Scale 1 on N(0,1) data: scores with a spread of about 11 per row, so a
    later tile's maximum often exceeds the running reference point by more
    than the kernel's slack and the accumulators are rescaled on many tiles;
    output and lse still match the oracle."""
    need_gpu()
    p = gi.small_prefill(1, 8, 2, 700, 128, seed=59)
    q, k, v = dev(p.q, "bf16"), dev(p.k, "bf16"), dev(p.v, "bf16")
    out, lse = gqa.gqa_prefill_causal(q, k, v, scale=1.0, return_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.prefill_causal(gi.to_f64(p.q, "bf16"), gi.to_f64(p.k, "bf16"),
                                         gi.to_f64(p.v, "bf16"), 1.0, return_lse=True)
    err, lerr = max_err(out.cpu().numpy(), ref), max_err(lse.cpu().numpy(), ref_lse)
    say("scale 1 max err", err, "lse err", lerr)
    assert err <= TOL["bf16"] and lerr <= TOL["bf16"]


def test_prefill_long_prompt_sampled_rows():
    """A 131,072-token causal prefill (B=1, Hq=4, Hkv=1, d=128; 4,096 q-tiles
    of one KV head): rows at tile and q-tile boundaries, the last rows and
    random rows of every head against the oracle's rows (row i attends keys
    0..i), output and lse."""
    need_gpu()
    N = 131072
    p = gi.small_prefill(1, 4, 1, N, 128, seed=5151)
    say("prefill long prompt", N)
    out, lse = run_prefill(p)
    rng = np.random.default_rng(7)
    rows = sorted({0, 1, 31, 32, 33, 63, 64, 65, 127, 128, 4095, 4096, 65535, 65536, N - 65, N - 64, N - 2, N - 1}
                  | set(int(r) for r in rng.integers(0, N, size=14)))
    k64, v64 = gi.to_f64(p.k[0], "bf16"), gi.to_f64(p.v[0], "bf16")
    worst = 0.0
    for h in range(4):
        ref, ref_lse = oracle.prefill_causal_rows(gi.to_f64(p.q[0, h, rows], "bf16"), k64, v64, rows, h, 4,
                                                  p.cfg.scale)
        worst = max(worst, max_err(out[0, h, rows], ref), max_err(lse[0, h, rows], ref_lse))
    say("max err over", len(rows), "rows x 4 heads", worst)
    assert worst <= TOL["bf16"]
