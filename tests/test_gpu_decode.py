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


def run_decode(inp, split_tokens=0, stages=False):
    """One decode call through the C ABI.

    stages=False: gqa_decode on a workspace that a call on other queries
    has just used, so it holds that call's partials (stale values that a
    read of an unwritten slot would pick up).
    stages=True: gqa_decode_split then gqa_decode_merge on a workspace filled
    with 0xFF bytes (NaN in every float slot), so unwritten partials show."""
    q, k, v, lens = decode_tensors(inp)
    B, Hq, d = q.shape
    Hkv, tcap = k.shape[1], k.shape[2]
    dt = gqa.GQA_BF16 if inp.cfg.dtype == "bf16" else gqa.GQA_F32
    plan = gqa.gqa_decode_plan(B, Hq, Hkv, d, tcap, dt, split_tokens)
    ws = gqa.decode_workspace(plan.workspace_bytes)
    if stages:
        ws.fill_(0xFF)
        out = torch.empty(B, Hq, d, dtype=torch.float32, device="cuda")
        gqa.gqa_decode_split(q, k, v, lens, out, ws, scale=inp.cfg.scale, split_tokens=split_tokens)
        gqa.gqa_decode_merge(lens, out, ws, Hkv, tcap, dt, split_tokens)
    else:
        gqa.gqa_decode(-q, k, v, lens, scale=inp.cfg.scale, workspace=ws, split_tokens=split_tokens)
        out = gqa.gqa_decode(q, k, v, lens, scale=inp.cfg.scale, workspace=ws, split_tokens=split_tokens)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle_full(inp):
    dt = inp.cfg.dtype
    return oracle.decode(gi.to_f64(inp.q, dt), gi.to_f64(inp.k_cache, dt), gi.to_f64(inp.v_cache, dt),
                         inp.seq_lens, inp.cfg.scale)


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
    ("bf16", 1, 71, 1, 128, [300], 320, 64),            # 71 heads on one KV head (5 blocks in 3 units)
    ("bf16", 2, 32, 1, 128, [900, 17], 960, 0),         # group 32: two full blocks share one unit
    ("bf16", 2, 40, 2, 64, [700, 1300], 1344, 128),     # group 20: a full block and a 4-head block
    ("bf16", 1, 48, 1, 128, [2000], 2048, 0),           # group 48: a two-block unit and a one-block unit
    ("bf16", 2, 128, 2, 128, [3000, 64], 3072, 0),      # group 64: two units of two blocks per KV head
    ("bf16", 2, 32, 2, 128, [4096, 1500], 4096, 0),     # group 16, wide
    # head_dim 64: up to five blocks (80 heads) share one unit
    ("bf16", 1, 71, 1, 64, [300], 320, 64),             # 71 heads: five blocks in one unit
    ("bf16", 2, 48, 1, 64, [1000, 77], 1024, 0),        # three blocks
    ("bf16", 2, 128, 2, 64, [700, 1300], 1344, 0),      # group 64 on two KV heads: four blocks
    ("bf16", 1, 96, 1, 64, [1500], 1536, 0),            # group 96: a five-block and a one-block unit
    ("bf16", 2, 80, 1, 64, [2048, 2048], 2048, 0),      # five full blocks, closed-form slot bases
    ("bf16", 3, 6, 2, 64, [0, 5, 64], 64, 0),           # empty sequence
    ("f32", 2, 8, 2, 64, [1, 300], 320, 64),
    ("f32", 2, 12, 3, 128, [129, 64], 192, 128),
    ("f32", 1, 20, 1, 64, [100], 128, 0),               # fp32, 20 heads on one (two head blocks)
    # equal lengths, range size left to the device; where the range size
    # divides the length, slot bases come from the closed form
    ("bf16", 4, 8, 2, 128, [1024] * 4, 1024, 0),        # closed form: 4 segments per unit
    ("bf16", 2, 8, 2, 128, [512, 512], 640, 0),         # closed form, padding past T
    ("bf16", 3, 32, 1, 64, [768] * 3, 768, 0),          # closed form, group 32 (two blocks per unit)
    ("bf16", 4, 8, 2, 128, [1000] * 4, 1024, 0),        # 256 does not divide 1000: stream scan
    ("bf16", 2, 8, 2, 128, [200, 200], 256, 0),         # shorter than one range: direct output, no merge
    ("bf16", 70, 8, 1, 64, [300] * 70, 320, 0),         # more than 64 sequences (block-wide scan)
    ("bf16", 40, 32, 16, 64, [256] * 40, 256, 0),       # 640 units on 512 workgroups: some take two
    ("bf16", 2, 64, 2, 128, [1500, 1500], 1536, 0),     # group 32, stream scan
    # many segments per unit: the merge takes several rounds of eight rows per thread
    ("bf16", 1, 8, 2, 64, [5000], 5120, 32),            # 157 segments, 128 per round at d = 64
    ("bf16", 1, 8, 2, 128, [4500], 4608, 32),           # 141 segments, 64 per round at d = 128
    ("f32", 1, 4, 1, 64, [3000], 3072, 32),             # 94 segments
]


@pytest.mark.parametrize("stages", [False, True], ids=["one-call", "two-stage"])
@pytest.mark.parametrize("case", SMALL_CASES, ids=lambda c: f"{c[0]}-B{c[1]}-{c[2]}on{c[3]}-d{c[4]}-split{c[7]}")
def test_small_shapes_full_parity(case, stages):
    need_gpu()
    dt, B, Hq, Hkv, d, lens, tcap, split = case
    inp = gi.small_decode(dt, B, Hq, Hkv, d, lens, tcap, seed=zlib.crc32(repr(case).encode()) % 100000)
    say("small", case, "two-stage" if stages else "one-call")
    got = run_decode(inp, split, stages)
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


_FULL = {}


def full_size_output(name):
    """GPU output of a full-size workload in the bench's launch configuration
    (gqa_decode, automatic ranges), computed once per test session."""
    if name not in _FULL:
        inp = gi.make_decode(gi.CONFIGS[name])
        say(name, gi.describe(inp.cfg), "sum T", int(inp.seq_lens.sum()))
        _FULL[name] = (inp, run_decode(inp))
    return _FULL[name]


def compare_sequences(inp, got, bs):
    """Every output row of sequences ``bs`` against oracle.decode, one
    sequence per call (the oracle repeats that sequence's K/V per head)."""
    dt = inp.cfg.dtype
    worst = 0.0
    for b in bs:
        T = int(inp.seq_lens[b])
        ref = oracle.decode(gi.to_f64(inp.q[b:b + 1], dt), gi.to_f64(inp.k_cache[b:b + 1, :, :T], dt),
                            gi.to_f64(inp.v_cache[b:b + 1, :, :T], dt), inp.seq_lens[b:b + 1], inp.cfg.scale)
        worst = max(worst, max_err(got[b:b + 1], ref))
    return worst


@pytest.mark.parametrize("part", range(4))
def test_wide_group_ragged_decode_full(part):
    """All 64 x 32 output rows of the wide-group workload, a quarter of the
    batch per test."""
    need_gpu()
    inp, got = full_size_output("wide-group")
    bs = range(16 * part, 16 * part + 16)
    err = compare_sequences(inp, got, bs)
    say("wide-group sequences", bs, "max err", err)
    assert err <= TOL["bf16"]


def test_mqa_128k_decode_full():
    """All 4 x 16 output rows of the mqa-128k workload."""
    need_gpu()
    inp, got = full_size_output("mqa-128k")
    err = compare_sequences(inp, got, range(inp.cfg.batch))
    say("mqa-128k max err", err)
    assert err <= TOL["bf16"]


def _mapping_probe(B, Hq, Hkv, T, split, d=128):
    """K = 0 and V constant per (b, KV head): V[...,0] = kv head, V[...,1] = b,
    V[...,2] = 1.  Every weight is exactly 1, so out[b,h,0] = h // g and
    out[b,h,1] = b exactly (sums stay below 2^24)."""
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


@pytest.mark.parametrize("B,Hq,Hkv,T,d", [(32, 32, 8, 8192, 128), (4, 16, 1, 4096, 128), (3, 71, 1, 64, 128),
                                             (2, 6, 2, 128, 128), (2, 96, 2, 256, 128), (2, 40, 1, 128, 128),
                                             (3, 71, 1, 64, 64), (2, 96, 2, 256, 64), (2, 170, 2, 96, 64)])
def test_mapping_probe_bit_exact(B, Hq, Hkv, T, d):
    need_gpu()
    say("mapping probe", B, Hq, Hkv, T, d)
    g = Hq // Hkv
    out = _mapping_probe(B, Hq, Hkv, T, split=((T + 63) // 64) * 64, d=d)   # one split: exact
    want_kv = np.array([h // g for h in range(Hq)], dtype=np.float32)
    assert np.array_equal(out[:, :, 0], np.broadcast_to(want_kv, (B, Hq)))
    assert np.array_equal(out[:, :, 1], np.broadcast_to(np.arange(B, dtype=np.float32)[:, None], (B, Hq)))
    assert np.all(out[:, :, 2] == 1.0) and np.all(out[:, :, 3:] == 0.0)
    multi = _mapping_probe(B, Hq, Hkv, T, split=64, d=d)   # merged splits: exact after rounding
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


def test_decode_at_largest_cache_capacity():
    """The largest cache the plan accepts at d = 128: 4,194,303 tokens per
    (sequence, KV head), the limit of one head's 32-bit byte offsets
    (T * d * 4 < 2^31).  Three sequences put the third one's rows more than
    2^31 bytes past the cache's base, so element offsets must be 64-bit; the
    lengths sit at and just below the capacity (the tail past each length is
    NaN), and each unit is split into hundreds of segments, which the merge
    combines in several rounds."""
    need_gpu()
    T = (2 ** 31 - 1) // (128 * 4)
    lens = [T, T - 1, T - 37]
    inp = gi.small_decode("bf16", 3, 1, 1, 128, lens, T, seed=4242)
    say("largest cache", T, "tokens x 3 sequences")
    got = run_decode(inp)
    for b in range(3):
        ref, _ = oracle.decode_one(gi.to_f64(inp.q[b, 0], "bf16"), gi.to_f64(inp.k_cache[b, :, :lens[b]], "bf16"),
                                   gi.to_f64(inp.v_cache[b, :, :lens[b]], "bf16"), lens[b], 0, 1, inp.cfg.scale)
        err = max_err(got[b, 0], ref)
        say("sequence", b, "max err", err)
        assert err <= TOL["bf16"]


@pytest.mark.parametrize("shape", [(3, 8, 2, 128), (2, 16, 1, 128), (2, 64, 2, 128), (2, 12, 3, 64)],
                         ids=lambda s: "B{}-{}on{}-d{}".format(*s))
def test_single_token_is_v0_bit_exact(shape):
    """A sequence holding one token: its only weight is 2^0 = 1 and the sum is
    1, so every query head of the group returns that token's V row exactly
    (the one-segment path writes it straight to the output); longer
    sequences in the same batch keep the tolerance."""
    need_gpu()
    B, Hq, Hkv, d = shape
    lens = [1] + [97 * (i + 1) for i in range(B - 1)]
    inp = gi.small_decode("bf16", B, Hq, Hkv, d, lens, 512, seed=zlib.crc32(repr(shape).encode()) % 100000)
    say("single token", shape, lens)
    got = run_decode(inp)
    g = Hq // Hkv
    for h in range(Hq):
        assert np.array_equal(got[0, h], gi.bf16_bits_to_f32(inp.v_cache[0, h // g, 0]))
    assert max_err(got, oracle_full(inp)) <= TOL["bf16"]


@pytest.mark.parametrize("split", [0, 64])
def test_zero_scale_gives_mean_of_v(split):
    """scale = 0: every attended token has weight 1, so each head returns the
    mean of its KV head's V rows over the sequence (a closed form that does
    not go through the oracle's softmax)."""
    need_gpu()
    lens = [1, 300, 1000]
    inp = gi.small_decode("bf16", 3, 16, 2, 128, lens, 1024, seed=777)
    q, k, v, sl = decode_tensors(inp)
    out = gqa.gqa_decode(q, k, v, sl, scale=0.0, split_tokens=split)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    vf = gi.to_f64(inp.v_cache, "bf16")
    for b, t in enumerate(lens):
        for h in range(16):
            mean = vf[b, h // 8, :t].mean(axis=0)
            assert np.max(np.abs(got[b, h] - mean)) <= 1e-3, (b, h)


def graph_replays_match_eager(step, out_graph, out_eager, disturb, replays=3):
    """Capture `step` (which writes out_graph) in a HIP graph and replay it:
    before each replay out_graph is NaN-filled outside the graph, after it the
    program's own eager work (`disturb`, which reuses the same workspace)
    runs with a synchronisation between, and every replay must equal the
    eager result bit for bit."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(replays):
        out_graph.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_graph, out_eager), f"replay {r}"
        disturb()
        torch.cuda.synchronize()


@pytest.mark.parametrize("split", [0, 64])
def test_decode_step_replays_from_a_hip_graph(split):
    """The decode step (split kernel and merge) launched with a caller-owned
    workspace can be captured in a HIP graph: the C call allocates nothing
    and records no memset, and the kernels rewrite every workspace byte they
    read, so replays after eager calls on other inputs are exact."""
    need_gpu()
    inp = gi.small_decode("bf16", 4, 32, 8, 128, [3000, 17, 4096, 1], 4096, seed=2929)
    q, k, v, lens = decode_tensors(inp)
    plan = gqa.gqa_decode_plan(4, 32, 8, 128, 4096, gqa.GQA_BF16, split)
    ws = gqa.decode_workspace(plan.workspace_bytes)
    say("graph replay, split", split, "workspace bytes", plan.workspace_bytes)
    out_e = gqa.gqa_decode(q, k, v, lens, scale=inp.cfg.scale, workspace=ws, split_tokens=split)
    torch.cuda.synchronize()
    assert max_err(out_e.cpu().numpy(), oracle_full(inp)) <= TOL["bf16"]
    out_g = torch.empty_like(out_e)
    out_x = torch.empty_like(out_e)
    graph_replays_match_eager(
        lambda: gqa.gqa_decode(q, k, v, lens, scale=inp.cfg.scale, out=out_g, workspace=ws, split_tokens=split),
        out_g, out_e,
        lambda: gqa.gqa_decode(q * 3, k, v, lens.flip(0).contiguous(), scale=inp.cfg.scale, out=out_x,
                               workspace=ws, split_tokens=split))
