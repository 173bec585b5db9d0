"""Decode over a batch in which no sequence holds a token.

A sequence of length 0 has an empty softmax; the library's reading is an
all-zero output row (the merge writes it, and no cache row is read).  With
every length 0 the split kernel finds no work at all, so these cases check
that every decode entry point still writes the whole output, exactly zero,
over an output and a workspace filled with NaN beforehand, and that no NaN
of the cache's padding reaches it."""
import numpy as np
import pytest
import torch

import gqa_inputs as gi
import grouped_query_attention_gqa_amd as gqa
from gpu_util import decode_tensors, dev, need_gpu, say

pytestmark = pytest.mark.gpu

B, HQ, HKV, TCAP = 3, 8, 2, 256


def nan_out(shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")


def assert_zero(out):
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got, np.zeros_like(got)), "non-zero output for an empty batch"


@pytest.mark.parametrize("dtype,d,split", [("bf16", 128, 0), ("bf16", 64, 64), ("f32", 64, 0), ("f32", 128, 32)])
def test_all_empty_decode_is_zero(dtype, d, split):
    need_gpu()
    inp = gi.small_decode(dtype, B, HQ, HKV, d, [0] * B, TCAP, seed=8100 + d)
    q, k, v, lens = decode_tensors(inp)
    dt = gqa.GQA_BF16 if dtype == "bf16" else gqa.GQA_F32
    plan = gqa.gqa_decode_plan(B, HQ, HKV, d, TCAP, dt, split)
    ws = gqa.decode_workspace(plan.workspace_bytes)
    say("empty batch", dtype, "d", d, "split", split)
    ws.fill_(0xFF)
    out = nan_out((B, HQ, d))
    gqa.gqa_decode(q, k, v, lens, scale=inp.cfg.scale, out=out, workspace=ws, split_tokens=split)
    assert_zero(out)
    # the two stages, on a workspace of NaN again
    ws.fill_(0xFF)
    out2 = nan_out((B, HQ, d))
    gqa.gqa_decode_split(q, k, v, lens, out2, ws, scale=inp.cfg.scale, split_tokens=split)
    gqa.gqa_decode_merge(lens, out2, ws, HKV, TCAP, dt, split)
    assert_zero(out2)


def test_all_empty_paged_and_fp8_decode_are_zero():
    need_gpu()
    inp = gi.small_decode("bf16", B, HQ, HKV, 128, [0] * B, TCAP, seed=8201)
    say("empty batch: paged and E4M3 caches")
    pg = gi.make_paged(inp, 16)
    q = dev(pg.q, "bf16")
    kp, vp = dev(pg.k_pages, "bf16"), dev(pg.v_pages, "bf16")
    bt = torch.from_numpy(pg.block_table).cuda()
    lens = torch.from_numpy(pg.seq_lens).cuda()
    plan = gqa.gqa_decode_plan(B, HQ, HKV, 128, bt.shape[1] * 16, gqa.GQA_BF16, 0)
    ws = gqa.decode_workspace(plan.workspace_bytes)
    ws.fill_(0xFF)
    out = gqa.gqa_decode_paged(q, kp, vp, bt, lens, scale=inp.cfg.scale, workspace=ws)
    assert_zero(out)

    fp = gi.make_fp8(inp)
    k8, v8 = torch.from_numpy(fp.k_cache).cuda(), torch.from_numpy(fp.v_cache).cuda()
    ks, vs = torch.from_numpy(fp.k_scale).cuda(), torch.from_numpy(fp.v_scale).cuda()
    plan = gqa.gqa_decode_plan(B, HQ, HKV, 128, TCAP, gqa.GQA_FP8_E4M3, 0)
    ws = gqa.decode_workspace(plan.workspace_bytes)
    ws.fill_(0xFF)
    out = gqa.gqa_decode_fp8(dev(fp.q, "bf16"), k8, v8, ks, vs, lens, scale=inp.cfg.scale, workspace=ws)
    assert_zero(out)


@pytest.mark.parametrize("split", [0, 32])
def test_all_empty_wide_decode_is_zero(split):
    need_gpu()
    w = gi.small_wide(2, 128, 1, 576, 512, [0, 0], 96, seed=8300 + split)
    say("empty batch: wide rows, split", split)
    out = gqa.gqa_decode_wide(dev(w.q, "bf16"), dev(w.kv_cache, "bf16"), torch.from_numpy(w.seq_lens).cuda(),
                              512, scale=w.cfg.scale, split_tokens=split)
    assert_zero(out)
