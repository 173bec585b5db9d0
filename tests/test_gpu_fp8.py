"""GPU decode over an FP8 (E4M3) cache through the C ABI, against the float64
FP8 oracle (exact dequantisation, then the plain decode)."""
import zlib

import numpy as np
import pytest
import torch

import gqa_inputs as gi
import grouped_query_attention_gqa_amd as gqa
import oracle
from gpu_util import TOL, dev, max_err, need_gpu, say

pytestmark = pytest.mark.gpu


def tensors(fp):
    return (dev(fp.q, "bf16"), torch.from_numpy(fp.k_cache).cuda(), torch.from_numpy(fp.v_cache).cuda(),
            torch.from_numpy(fp.k_scale).cuda(), torch.from_numpy(fp.v_scale).cuda(),
            torch.from_numpy(fp.seq_lens).cuda())


def run_fp8(fp, split_tokens=0, v_scale=None):
    q, k, v, ks, vs, lens = tensors(fp)
    if v_scale is not None:
        vs = torch.from_numpy(v_scale).cuda()
    B, Hq, d = q.shape
    plan = gqa.gqa_decode_plan(B, Hq, k.shape[1], d, k.shape[2], gqa.GQA_FP8_E4M3, split_tokens)
    ws = gqa.decode_workspace(plan.workspace_bytes)
    # a call on other queries first: the workspace then holds stale partials
    gqa.gqa_decode_fp8(-q, k, v, ks, vs, lens, scale=fp.cfg.scale, workspace=ws, split_tokens=split_tokens)
    out = gqa.gqa_decode_fp8(q, k, v, ks, vs, lens, scale=fp.cfg.scale, workspace=ws, split_tokens=split_tokens)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def fp8_oracle(fp):
    return oracle.decode_fp8(gi.to_f64(fp.q, "bf16"), fp.k_cache, fp.v_cache, fp.k_scale, fp.v_scale,
                             fp.seq_lens, fp.cfg.scale)


CASES = [
    # B, Hq, Hkv, d, lens, T_cap, split
    (3, 32, 8, 128, [300, 1, 1023], 1024, 0),
    (2, 16, 1, 128, [4096, 77], 4096, 0),
    (4, 8, 2, 64, [0, 5, 129, 64], 192, 64),
    (2, 32, 2, 128, [2000, 513], 2048, 256),
    (1, 71, 1, 128, [333], 512, 64),
    (2, 64, 2, 128, [1500, 40], 1536, 0),     # group 32: two head blocks per unit
    (2, 40, 1, 64, [700, 129], 768, 128),     # group 40: a two-block unit and an 8-head unit
    (2, 12, 3, 64, [33, 250], 256, 0),
    (1, 71, 1, 64, [900], 1024, 0),           # head_dim 64: 71 heads, five blocks in one unit
    (2, 64, 1, 64, [500, 333], 512, 64),      # four blocks
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}-{}on{}-d{}-split{}".format(c[0], c[1], c[2], c[3], c[6]))
def test_fp8_small_full_parity(case):
    need_gpu()
    B, Hq, Hkv, d, lens, T, split = case
    inp = gi.small_decode("bf16", B, Hq, Hkv, d, lens, T, seed=zlib.crc32(repr(case).encode()) % 100000)
    fp = gi.make_fp8(inp)
    say("fp8 small", case)
    got = run_fp8(fp, split)
    err = max_err(got, fp8_oracle(fp))
    say("max err", err)
    assert err <= TOL["bf16"]


def test_fp8_two_stage_matches_oracle():
    """gqa_decode_fp8_split + gqa_decode_merge on a workspace of 0xFF bytes
    (NaN in every float slot, so unwritten partials would show)."""
    need_gpu()
    inp = gi.small_decode("bf16", 3, 32, 2, 128, [2000, 1, 513], 2048, seed=97)
    fp = gi.make_fp8(inp)
    q, k, v, ks, vs, lens = tensors(fp)
    for split in (0, 64):
        plan = gqa.gqa_decode_plan(3, 32, 2, 128, 2048, gqa.GQA_FP8_E4M3, split)
        ws = gqa.decode_workspace(plan.workspace_bytes)
        ws.fill_(0xFF)
        out = gqa.gqa_decode_fp8(q, k, v, ks, vs, lens, scale=fp.cfg.scale, workspace=ws, split_tokens=split,
                                 stage="split")
        gqa.gqa_decode_merge(lens, out, ws, 2, 2048, gqa.GQA_FP8_E4M3, split)
        torch.cuda.synchronize()
        assert max_err(out.cpu().numpy(), fp8_oracle(fp)) <= TOL["bf16"], split


def test_fp8_llama3_8b_full_size():
    """All 32 x 32 output rows of the llama3-8b workload over its E4M3 cache,
    one sequence per oracle call."""
    need_gpu()
    cfg = gi.CONFIGS["llama3-8b"]
    fp = gi.make_fp8(gi.make_decode(cfg))
    say("fp8", gi.describe(cfg))
    got = run_fp8(fp)
    worst = 0.0
    for b in range(cfg.batch):
        ref = oracle.decode_fp8(gi.to_f64(fp.q[b:b + 1], "bf16"), fp.k_cache[b:b + 1], fp.v_cache[b:b + 1],
                                fp.k_scale, fp.v_scale, fp.seq_lens[b:b + 1], cfg.scale)
        worst = max(worst, max_err(got[b:b + 1], ref))
    say("fp8 llama3-8b max err", worst)
    assert worst <= TOL["bf16"]


def test_fp8_v_scale_is_exact_output_scale():
    """Doubling every V scale doubles the output bit for bit (a power-of-two
    factor on the normalised output and on every merged partial)."""
    need_gpu()
    inp = gi.small_decode("bf16", 2, 16, 4, 128, [900, 350], 1024, seed=23)
    fp = gi.make_fp8(inp)
    a = run_fp8(fp, 64)
    b = run_fp8(fp, 64, v_scale=fp.v_scale * 2)
    assert np.array_equal(b, 2 * a)


def test_fp8_mapping_probe_bit_exact():
    """K codes 0 make every weight 1; V codes hold (kv head, sequence, 1) with
    unit scales, so out[..., 0] = h // g and out[..., 1] = b exactly."""
    need_gpu()
    B, Hq, Hkv, d, T = 3, 24, 6, 128, 256
    inp = gi.small_decode("bf16", B, Hq, Hkv, d, [T] * B, T, seed=29)
    fp = gi.make_fp8(inp)
    fp.k_cache[...] = 0
    fp.v_cache[...] = 0
    for b in range(B):
        for kv in range(Hkv):
            fp.v_cache[b, kv, :, :3] = gi.f32_to_e4m3_bits(np.array([kv, b, 1.0]))
    fp.k_scale[:] = 1.0
    fp.v_scale[:] = 1.0
    got = run_fp8(fp, split_tokens=T)
    g = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            assert got[b, h, 0] == h // g and got[b, h, 1] == b and got[b, h, 2] == 1, (b, h)
    assert np.all(got[:, :, 3:] == 0)


def test_fp8_rejected_by_bf16_entry_points():
    need_gpu()
    q = torch.zeros(1, 8, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 2, 64, 128, dtype=torch.bfloat16, device="cuda")
    lens = torch.full((1,), 64, dtype=torch.int32, device="cuda")
    lib = gqa.load_library()
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    out = torch.empty(1, 8, 128, device="cuda")
    st = lib.gqa_decode(q.data_ptr(), k.data_ptr(), k.data_ptr(), lens.data_ptr(), out.data_ptr(), 1, 8, 2, 128,
                        64, 0.1, gqa.GQA_FP8_E4M3, 0, ws.data_ptr(), ws.numel(), None)
    assert st == 3   # GQA_ERR_UNSUPPORTED
