"""GPU decode (split-K kernels through the C ABI) against the float64 oracle."""
import zlib

import numpy as np
import pytest
import torch

import gqa_inputs as gi
import grouped_query_attention_gqa_amd as gqa
import oracle
from gpu_util import TOL, decode_tensors, dev, max_err, need_gpu, say

pytestmark = pytest.mark.gpu


def run_decode(inp, split_tokens=0, poison_workspace=True):
    q, k, v, lens = decode_tensors(inp)
    B, Hq, d = q.shape
    plan = gqa.gqa_decode_plan(B, Hq, k.shape[1], d, k.shape[2],
                               gqa.GQA_BF16 if inp.cfg.dtype == "bf16" else gqa.GQA_F32, split_tokens)
    ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    if poison_workspace:
        ws.fill_(0xFF)   # NaN in every float slot: unwritten partials would show
    out = gqa.gqa_decode(q, k, v, lens, scale=inp.cfg.scale, workspace=ws, split_tokens=split_tokens)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle_full(inp):
    dt = inp.cfg.dtype
    return oracle.decode(gi.to_f64(inp.q, dt), gi.to_f64(inp.k_cache, dt), gi.to_f64(inp.v_cache, dt),
                         inp.seq_lens, inp.cfg.scale)


def check_rows(inp, got, pairs):
    """Compare sampled (b, h) rows one by one against the oracle."""
    dt = inp.cfg.dtype
    worst = 0.0
    for b, h in pairs:
        ref, _ = oracle.decode_one(gi.to_f64(inp.q[b, h], dt), inp.k_cache[b] if dt == "f32" else
                                   gi.bf16_bits_to_f32(inp.k_cache[b, :, :inp.seq_lens[b]]),
                                   inp.v_cache[b] if dt == "f32" else
                                   gi.bf16_bits_to_f32(inp.v_cache[b, :, :inp.seq_lens[b]]),
                                   inp.seq_lens[b], h, inp.cfg.num_q_heads, inp.cfg.scale)
        worst = max(worst, max_err(got[b, h], ref))
    return worst


def test_tiny_fp32_decode_full_parity():
    need_gpu()
    inp = gi.make_decode(gi.CONFIGS["tiny-f32"])
    say("tiny-f32", gi.describe(inp.cfg))
    err = max_err(run_decode(inp), oracle_full(inp))
    say("tiny-f32 max err", err)
    assert err <= TOL["f32"]


SMALL_CASES = [
    # dtype, B, Hq, Hkv, d, lens, tcap, split
    ("bf16", 3, 8, 2, 128, [1, 100, 1000], 1024, 0),
    ("bf16", 3, 8, 2, 128, [1, 100, 1000], 1024, 64),
    ("bf16", 3, 8, 2, 128, [33, 257, 1000], 1024, 256),
    ("bf16", 2, 8, 2, 64, [77, 640], 640, 128),
    ("bf16", 2, 4, 4, 128, [500, 129], 512, 128),       # MHA endpoint
    ("bf16", 2, 16, 1, 128, [700, 31], 704, 192),       # MQA, group 16
    ("bf16", 1, 71, 1, 128, [300], 320, 64),            # 71 heads on one KV head (5 head blocks)
    ("bf16", 2, 32, 2, 128, [4096, 1500], 4096, 0),     # group 16, wide
    ("bf16", 3, 6, 2, 64, [0, 5, 64], 64, 0),           # empty sequence
    ("f32", 2, 8, 2, 64, [1, 300], 320, 64),
    ("f32", 2, 12, 3, 128, [129, 64], 192, 128),
    ("f32", 1, 20, 1, 64, [100], 128, 0),               # fp32, 20 heads on one (two head blocks)
    # many segments per unit: the merge takes several rounds of eight rows per thread
    ("bf16", 1, 8, 2, 64, [5000], 5120, 32),            # 157 segments, 128 per round at d = 64
    ("bf16", 1, 8, 2, 128, [4500], 4608, 32),           # 141 segments, 64 per round at d = 128
    ("f32", 1, 4, 1, 64, [3000], 3072, 32),             # 94 segments
]


@pytest.mark.parametrize("case", SMALL_CASES, ids=lambda c: f"{c[0]}-B{c[1]}-{c[2]}on{c[3]}-d{c[4]}-split{c[7]}")
def test_small_shapes_full_parity(case):
    need_gpu()
    dt, B, Hq, Hkv, d, lens, tcap, split = case
    inp = gi.small_decode(dt, B, Hq, Hkv, d, lens, tcap, seed=zlib.crc32(repr(case).encode()) % 100000)
    say("small", case)
    got = run_decode(inp, split)
    ref = oracle_full(inp)
    err = max_err(got, ref)
    say("max err", err)
    assert err <= TOL[dt]
    for b, t in enumerate(lens):
        if t == 0:
            assert np.all(got[b] == 0.0)


def test_llama3_8b_decode_full_parity():
    need_gpu()
    inp = gi.make_decode(gi.CONFIGS["llama3-8b"])
    say("llama3-8b", gi.describe(inp.cfg))
    got = run_decode(inp)
    err = max_err(got, oracle_full(inp))
    say("llama3-8b max err", err)
    assert err <= TOL["bf16"]


def test_wide_group_ragged_decode_sampled():
    need_gpu()
    inp = gi.make_decode(gi.CONFIGS["wide-group"])
    say("wide-group", gi.describe(inp.cfg), "sum T", int(inp.seq_lens.sum()))
    got = run_decode(inp)
    lens = inp.seq_lens
    bs = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 0, 17, 40, 63})
    pairs = [(b, h) for b in bs for h in (0, 1, 15, 16, 17, 31)]
    err = check_rows(inp, got, pairs)
    say("wide-group sampled max err", err)
    assert err <= TOL["bf16"]
    # all rows: finite and inside the hull of the attended values (per coordinate)
    assert np.all(np.isfinite(got))


def test_mqa_128k_decode_sampled():
    need_gpu()
    inp = gi.make_decode(gi.CONFIGS["mqa-128k"])
    say("mqa-128k", gi.describe(inp.cfg))
    got = run_decode(inp)
    pairs = [(b, h) for b in range(4) for h in (0, 5, 15)] + [(0, h) for h in range(16)]
    err = check_rows(inp, got, sorted(set(pairs)))
    say("mqa-128k sampled max err", err)
    assert err <= TOL["bf16"]


def _mapping_probe(B, Hq, Hkv, T, split):
    """K = 0 and V constant per (b, KV head): V[...,0] = kv head, V[...,1] = b,
    V[...,2] = 1.  Every weight is exactly 1, so out[b,h,0] = h // g and
    out[b,h,1] = b exactly (sums stay below 2^24)."""
    d = 128
    k = torch.zeros(B, Hkv, T, d, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros(B, Hkv, T, d, dtype=torch.float32)
    v[..., 0] = torch.arange(Hkv, dtype=torch.float32)[None, :, None]
    v[..., 1] = torch.arange(B, dtype=torch.float32)[:, None, None]
    v[..., 2] = 1.0
    v = v.to(torch.bfloat16).cuda()
    q = torch.randn(B, Hq, d, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16).cuda()
    lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
    out = gqa.gqa_decode(q, k, v, lens, split_tokens=split)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("B,Hq,Hkv,T", [(32, 32, 8, 8192), (4, 16, 1, 4096), (3, 71, 1, 64), (2, 6, 2, 128)])
def test_mapping_probe_bit_exact(B, Hq, Hkv, T):
    need_gpu()
    say("mapping probe", B, Hq, Hkv, T)
    g = Hq // Hkv
    out = _mapping_probe(B, Hq, Hkv, T, split=((T + 63) // 64) * 64)   # one split: exact
    want_kv = np.array([h // g for h in range(Hq)], dtype=np.float32)
    assert np.array_equal(out[:, :, 0], np.broadcast_to(want_kv, (B, Hq)))
    assert np.array_equal(out[:, :, 1], np.broadcast_to(np.arange(B, dtype=np.float32)[:, None], (B, Hq)))
    assert np.all(out[:, :, 2] == 1.0) and np.all(out[:, :, 3:] == 0.0)
    multi = _mapping_probe(B, Hq, Hkv, T, split=64)        # merged splits: exact after rounding
    assert np.array_equal(np.rint(multi[:, :, 0]), out[:, :, 0])
    assert np.array_equal(np.rint(multi[:, :, 1]), out[:, :, 1])


def test_single_token_returns_v0_exactly():
    need_gpu()
    inp = gi.small_decode("bf16", 2, 8, 2, 128, [1, 1], 64, seed=5)
    got = run_decode(inp)
    for b in range(2):
        for h in range(8):
            assert np.array_equal(got[b, h], gi.bf16_bits_to_f32(inp.v_cache[b, h // 4, 0]))


def test_split_invariance_and_determinism():
    need_gpu()
    inp = gi.small_decode("bf16", 2, 32, 8, 128, [2048, 1999], 2048, seed=9)
    a = run_decode(inp, split_tokens=2048)
    b = run_decode(inp, split_tokens=64)
    c = run_decode(inp, split_tokens=64)
    assert max_err(a, b.astype(np.float64)) <= 1e-3
    assert np.array_equal(b, c)   # run twice: bitwise identical


def test_decode_matches_prefill_last_row():
    need_gpu()
    p = gi.small_prefill(1, 8, 2, 300, 128, seed=12)
    q, k, v = dev(p.q, "bf16"), dev(p.k, "bf16"), dev(p.v, "bf16")
    pre = gqa.gqa_prefill_causal(q, k, v)
    lens = torch.tensor([300], dtype=torch.int32, device="cuda")
    dec = gqa.gqa_decode(q[:, :, -1].contiguous(), k, v, lens)
    torch.cuda.synchronize()
    assert max_err(dec.cpu().numpy(), pre[:, :, -1].cpu().numpy().astype(np.float64)) <= 2e-2
