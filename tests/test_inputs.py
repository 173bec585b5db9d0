"""The seeded input generator (CPU only)."""
import numpy as np
import torch

import gqa_inputs as gi


def test_bf16_rounding_matches_torch_rne():
    r = np.random.default_rng(5)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32),
                        np.array([1.0, -2.5, 3.0e-3, 65504.0, 1.00390625, 1.01171875], dtype=np.float32)])
    ours = gi.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = gi.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_decode_inputs_deterministic_and_shaped():
    cfg = gi.CONFIGS["tiny-f32"]
    a = gi.make_decode(cfg)
    b = gi.make_decode(cfg)
    assert a.q.shape == (1, 8, 64) and a.k_cache.shape == (1, 2, 256, 64)
    assert a.q.dtype == np.float32
    for x, y in [(a.q, b.q), (a.k_cache, b.k_cache), (a.v_cache, b.v_cache), (a.seq_lens, b.seq_lens)]:
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))
    assert a.seq_lens.tolist() == [256]
    # distinct K per KV head and distinct Q per query head
    assert not np.array_equal(a.k_cache[0, 0], a.k_cache[0, 1])
    assert len({a.q[0, h].tobytes() for h in range(8)}) == 8


def test_ragged_lengths_and_padding():
    cfg = gi.CONFIGS["wide-group"]
    lens = gi.make_seq_lens(cfg)
    assert lens.dtype == np.int32 and lens.shape == (64,)
    assert lens.min() >= 1024 and lens.max() <= 32768
    assert len(set(lens.tolist())) > 50
    small = gi.small_decode("bf16", 3, 4, 2, 64, [5, 0, 9], 12, 77)
    for b, t in enumerate([5, 0, 9]):
        assert np.all(small.k_cache[b, :, t:] == gi.BF16_NAN_BITS)
        assert np.all(small.v_cache[b, :, t:] == gi.BF16_NAN_BITS)
        assert np.all(np.isfinite(gi.bf16_bits_to_f32(small.k_cache[b, :, :t])))


def test_prefill_inputs():
    p = gi.small_prefill(1, 4, 2, 33, 128, 9)
    assert p.q.shape == (1, 4, 33, 128) and p.k.shape == (1, 2, 33, 128) and p.q.dtype == np.uint16
    f = gi.to_f64(p.q, "bf16")
    assert abs(f.mean()) < 0.05 and abs(f.std() - 1.0) < 0.05


def test_workload_table():
    c = gi.CONFIGS
    assert (c["llama3-8b"].batch, c["llama3-8b"].num_q_heads, c["llama3-8b"].num_kv_heads, c["llama3-8b"].head_dim, c["llama3-8b"].max_seq_len) == (32, 32, 8, 128, 8192)
    assert (c["mqa-128k"].batch, c["mqa-128k"].num_q_heads, c["mqa-128k"].num_kv_heads, c["mqa-128k"].max_seq_len) == (4, 16, 1, 131072)
    assert (c["prefill-4k"].batch, c["prefill-4k"].num_q_heads, c["prefill-4k"].num_kv_heads, c["prefill-4k"].seq_len) == (2, 32, 8, 4096)
    assert [c[k].seed for k in ("tiny-f32", "llama3-8b", "wide-group", "mqa-128k", "prefill-4k")] == [1001, 1002, 1003, 1004, 1005]


def test_wide_inputs():
    cfg = gi.WIDE_CONFIGS["mla-decode"]
    assert (cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.d_k, cfg.d_v, cfg.max_len, cfg.seed) == \
        (64, 128, 1, 576, 512, 4096, 1006)
    assert abs(cfg.scale - 1 / 192 ** 0.5) < 1e-15
    a = gi.small_wide(2, 8, 1, 576, 512, [40, 7], 48, seed=5)
    b = gi.small_wide(2, 8, 1, 576, 512, [40, 7], 48, seed=5)
    assert a.q.shape == (2, 8, 576) and a.kv_cache.shape == (2, 1, 48, 576) and a.q.dtype == np.uint16
    assert np.array_equal(a.q, b.q) and np.array_equal(a.kv_cache, b.kv_cache)
    assert np.all(a.kv_cache[1, :, 7:] == gi.BF16_NAN_BITS)
    assert np.all(np.isfinite(gi.bf16_bits_to_f32(a.kv_cache[1, :, :7])))
