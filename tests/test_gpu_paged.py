"""GPU decode over a paged KV cache (through the C ABI) against the float64
paged oracle, and against the contiguous GPU path on the same values."""
import zlib

import numpy as np
import pytest
import torch

import gqa_inputs as gi
import grouped_query_attention_gqa_amd as gqa
import oracle
from gpu_util import TOL, dev, max_err, need_gpu, say

pytestmark = pytest.mark.gpu


def run_paged(pg, split_tokens=0, table=None):
    q = dev(pg.q, "bf16")
    kp, vp = dev(pg.k_pages, "bf16"), dev(pg.v_pages, "bf16")
    bt = torch.from_numpy(pg.block_table if table is None else table).cuda()
    lens = torch.from_numpy(pg.seq_lens).cuda()
    B, Hq, d = q.shape
    plan = gqa.gqa_decode_plan(B, Hq, kp.shape[1], d, bt.shape[1] * pg.page_size, gqa.GQA_BF16, split_tokens)
    ws = gqa.decode_workspace(plan.workspace_bytes)
    # a call on other queries first: the workspace then holds stale partials
    gqa.gqa_decode_paged(-q, kp, vp, bt, lens, scale=pg.cfg.scale, workspace=ws, split_tokens=split_tokens)
    out = gqa.gqa_decode_paged(q, kp, vp, bt, lens, scale=pg.cfg.scale, workspace=ws,
                               split_tokens=split_tokens)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def run_contiguous(inp, split_tokens=0):
    q, k, v = dev(inp.q, "bf16"), dev(inp.k_cache, "bf16"), dev(inp.v_cache, "bf16")
    lens = torch.from_numpy(inp.seq_lens).cuda()
    out = gqa.gqa_decode(q, k, v, lens, scale=inp.cfg.scale, split_tokens=split_tokens)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def paged_oracle(pg):
    return oracle.decode_paged(gi.to_f64(pg.q, "bf16"), gi.to_f64(pg.k_pages, "bf16"),
                               gi.to_f64(pg.v_pages, "bf16"), pg.block_table, pg.seq_lens,
                               pg.page_size, pg.cfg.scale)


CASES = [
    # B, Hq, Hkv, d, lens, T_cap, page_size
    (3, 32, 8, 128, [300, 1, 1023], 1024, 16),
    (2, 16, 1, 128, [4096, 77], 4096, 64),
    (4, 8, 2, 64, [0, 5, 129, 64], 192, 32),
    (2, 32, 2, 128, [2000, 513], 2048, 256),
    (1, 4, 4, 128, [97], 128, 1),          # one token per page
    (2, 12, 3, 64, [33, 250], 256, 8),     # group 4 of 12, pages smaller than a tile
    (2, 64, 2, 128, [1000, 333], 1024, 16),  # group 32: two head blocks per unit
    (1, 48, 1, 64, [777], 800, 32),        # group 48 at head_dim 64: three blocks in one unit
    (2, 71, 1, 64, [600, 129], 640, 16),   # 71 heads at head_dim 64: five blocks in one unit
    (1, 128, 2, 64, [1000], 1024, 64),     # group 64 at head_dim 64: four blocks
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}-{}on{}-d{}-ps{}".format(c[0], c[1], c[2], c[3], c[6]))
def test_paged_small_full_parity(case):
    need_gpu()
    B, Hq, Hkv, d, lens, T, ps = case
    inp = gi.small_decode("bf16", B, Hq, Hkv, d, lens, T, seed=zlib.crc32(repr(case).encode()) % 100000)
    pg = gi.make_paged(inp, page_size=ps, seed=ps + 1)
    say("paged small", case, "pool pages", pg.k_pages.shape[0])
    got = run_paged(pg)
    err = max_err(got, paged_oracle(pg))
    say("max err", err)
    assert err <= TOL["bf16"]
    # the same values read contiguously give bit-identical results
    assert np.array_equal(got, run_contiguous(inp))


def test_paged_forced_splits_match_contiguous():
    need_gpu()
    inp = gi.small_decode("bf16", 2, 16, 2, 128, [3000, 1500], 3072, seed=91)
    pg = gi.make_paged(inp, page_size=16, seed=3)
    for split in (32, 256, 4096):
        got = run_paged(pg, split_tokens=split)
        assert max_err(got, paged_oracle(pg)) <= TOL["bf16"], split
        assert np.array_equal(got, run_contiguous(inp, split_tokens=split)), split


def test_paged_two_stage_matches_oracle():
    """gqa_decode_paged_split + gqa_decode_merge on a workspace of 0xFF bytes
    (NaN in every float slot, so unwritten partials would show)."""
    need_gpu()
    inp = gi.small_decode("bf16", 3, 16, 2, 128, [3000, 1, 700], 3072, seed=93)
    pg = gi.make_paged(inp, page_size=16, seed=8)
    q = dev(pg.q, "bf16")
    kp, vp = dev(pg.k_pages, "bf16"), dev(pg.v_pages, "bf16")
    bt, lens = torch.from_numpy(pg.block_table).cuda(), torch.from_numpy(pg.seq_lens).cuda()
    tcap = bt.shape[1] * pg.page_size
    for split in (0, 64):
        plan = gqa.gqa_decode_plan(3, 16, 2, 128, tcap, gqa.GQA_BF16, split)
        ws = gqa.decode_workspace(plan.workspace_bytes)
        ws.fill_(0xFF)
        out = gqa.gqa_decode_paged(q, kp, vp, bt, lens, scale=pg.cfg.scale, workspace=ws, split_tokens=split,
                                   stage="split")
        gqa.gqa_decode_merge(lens, out, ws, 2, tcap, gqa.GQA_BF16, split)
        torch.cuda.synchronize()
        assert max_err(out.cpu().numpy(), paged_oracle(pg)) <= TOL["bf16"], split


def test_paged_llama3_8b_full_size():
    need_gpu()
    cfg = gi.CONFIGS["llama3-8b"]
    inp = gi.make_decode(cfg)
    pg = gi.make_paged(inp, page_size=16, seed=17)
    say("paged", gi.describe(cfg), "page_size 16, pool pages", pg.k_pages.shape[0])
    got = run_paged(pg)
    assert np.all(np.isfinite(got))
    assert np.array_equal(got, run_contiguous(inp))
    kp, vp = gi.to_f64(pg.k_pages, "bf16"), gi.to_f64(pg.v_pages, "bf16")
    worst = 0.0
    for b in range(cfg.batch):   # every output row, one sequence per oracle call
        ref = oracle.decode_paged(gi.to_f64(pg.q[b:b + 1], "bf16"), kp, vp, pg.block_table[b:b + 1],
                                  pg.seq_lens[b:b + 1], pg.page_size, cfg.scale)
        worst = max(worst, max_err(got[b:b + 1], ref))
    say("paged llama3-8b max err", worst)
    assert worst <= TOL["bf16"]


def _probe_inputs(lens, T, B=3, Hq=24, Hkv=6, d=64):
    inp = gi.small_decode("bf16", B, Hq, Hkv, d, lens, T, seed=101)
    inp.k_cache[...] = 0
    for b in range(B):
        for kv in range(Hkv):
            row = np.zeros(d, dtype=np.float32)
            row[:3] = (kv, b, 1)
            inp.v_cache[b, kv, :] = gi.f32_to_bf16_bits(row)
    return inp


def test_paged_mapping_probe_bit_exact():
    """K = 0 makes every weight 1; V = (kv head, sequence, 1) in every row of
    every page, so out[..., 0] and out[..., 1] are exactly h // g and b when
    each sequence is one range (and after rounding when ranges are merged)."""
    need_gpu()
    Hq, Hkv = 24, 6
    g = Hq // Hkv
    want_kv = np.array([h // g for h in range(Hq)], dtype=np.float32)
    pg = gi.make_paged(_probe_inputs([192, 192, 192], 192), page_size=16, seed=4)
    got = run_paged(pg, split_tokens=192)
    assert np.array_equal(got[:, :, 0], np.broadcast_to(want_kv, (3, Hq)))
    assert np.array_equal(got[:, :, 1], np.broadcast_to(np.arange(3, dtype=np.float32)[:, None], (3, Hq)))
    assert np.all(got[:, :, 2] == 1.0) and np.all(got[:, :, 3:] == 0.0)
    pg = gi.make_paged(_probe_inputs([200, 37, 1], 208), page_size=16, seed=5)
    got = run_paged(pg, split_tokens=64)
    assert np.array_equal(np.rint(got[:, :, 0]), np.broadcast_to(want_kv, (3, Hq)))
    assert np.array_equal(np.rint(got[:, :, 1]), np.broadcast_to(np.arange(3, dtype=np.float32)[:, None], (3, Hq)))


def test_out_of_range_table_entries_are_contained():
    """Entries outside the pool are clamped into it: the call completes (its
    output is not meaningful) and a following valid call is still exact."""
    need_gpu()
    inp = gi.small_decode("bf16", 2, 8, 2, 128, [100, 60], 128, seed=7)
    pg = gi.make_paged(inp, page_size=16, seed=2)
    bad = pg.block_table.copy()
    bad[0, 1] = 1 << 30
    bad[1, 0] = -5
    run_paged(pg, table=bad)
    got = run_paged(pg)
    assert max_err(got, paged_oracle(pg)) <= TOL["bf16"]
