"""Pins of the wide-row (absorbed-MLA) decode oracle (oracle/wide.py).

Each pin takes the module so test_oracle_wide.py can run them against broken
copies too.  They check the oracle against the equivalence the MLA passage
of anrans.github.io ("Attention variants: MQA, GQA, MLA", section "MLA:
multi-head latent attention") asserts: per-head attention over keys and
values rebuilt from the latent vectors, with a shared rotary key, equals
attention of the absorbed query against the cached latent rows followed by
the value up-projection.  Further: a scalar brute force, the pinned decode
oracle when the value is the whole row, uniform weights at scale 0, and the
rotary columns acting only through the scores."""
import math

import numpy as np

import gqa_inputs as gi
import oracle
from brute import brute_decode


def pin_absorption_equivalence(w):
    """The MLA weight-absorption identity with decoupled rotary dimensions:
    naive per-head attention (K, V rebuilt from the latent cache, written
    out with scalar loops) against decode_wide on [latent | rotary key] rows
    with the absorbed query, then W_UV per head."""
    rng = np.random.default_rng(17)
    T, d_model, d_c, n_h, d_h, d_r = 7, 64, 16, 4, 8, 4
    h = rng.standard_normal((T, d_model))
    W_q = rng.standard_normal((d_model, n_h * d_h)) / 8
    W_qr = rng.standard_normal((d_model, n_h * d_r)) / 8
    W_dkv = rng.standard_normal((d_model, d_c)) / 8
    W_kr = rng.standard_normal((d_model, d_r)) / 8
    W_uk = rng.standard_normal((n_h, d_c, d_h)) / 4
    W_uv = rng.standard_normal((n_h, d_c, d_h)) / 4
    c = h @ W_dkv                              # the latent cache [T, d_c]
    k_rope = h @ W_kr                          # shared rotary key [T, d_r]
    qn = (h[-1] @ W_q).reshape(n_h, d_h)       # the newest token's query
    qr = (h[-1] @ W_qr).reshape(n_h, d_r)
    scale = 1.0 / math.sqrt(d_h + d_r)
    naive = np.zeros((n_h, d_h))
    for i in range(n_h):
        k_i = c @ W_uk[i]
        v_i = c @ W_uv[i]
        s = [scale * (float(qn[i] @ k_i[t]) + float(qr[i] @ k_rope[t])) for t in range(T)]
        top = max(s)
        wts = [math.exp(x - top) for x in s]
        tot = math.fsum(wts)
        for col in range(d_h):
            naive[i, col] = math.fsum(wt * v_i[t, col] for t, wt in enumerate(wts)) / tot
    q_abs = np.concatenate([np.stack([W_uk[i] @ qn[i] for i in range(n_h)]), qr], axis=1)   # [n_h, d_c+d_r]
    rows = np.concatenate([c, k_rope], axis=1)                                             # [T, d_c+d_r]
    lat = w.decode_wide(q_abs[None], rows[None, None], np.array([T]), d_c, scale)[0]       # [n_h, d_c]
    absorbed = np.stack([lat[i] @ W_uv[i] for i in range(n_h)])
    assert np.max(np.abs(absorbed - naive)) <= 1e-12


def pin_wide_brute(w):
    """Scalar brute force with values = the leading columns of each row, on
    a group of 3 over two KV heads with ragged lengths."""
    inp = gi.small_wide(2, 6, 2, 12, 8, [5, 3], 6, seed=301)
    q, kv = gi.to_f64(inp.q, "bf16"), gi.to_f64(inp.kv_cache, "bf16")
    got = w.decode_wide(q, kv, inp.seq_lens, 8, 0.3)
    ref = np.asarray(brute_decode(q.tolist(), kv.tolist(), kv[..., :8].tolist(), inp.seq_lens.tolist(), 0.3))
    assert np.max(np.abs(got - ref)) <= 1e-12


def pin_whole_row_value_is_decode(w):
    """With d_v = d_k the row is K and V at once: the pinned decode oracle
    with v = k."""
    inp = gi.small_wide(2, 8, 1, 16, 16, [9, 4], 10, seed=307)
    q, kv = gi.to_f64(inp.q, "bf16"), gi.to_f64(inp.kv_cache, "bf16")
    got, lse = w.decode_wide(q, kv, inp.seq_lens, 16, 0.25, return_lse=True)
    ref, ref_lse = oracle.decode(q, kv, kv, inp.seq_lens, 0.25, return_lse=True)
    assert np.max(np.abs(got - ref)) <= 1e-13 and np.max(np.abs(lse - ref_lse)) <= 1e-13


def pin_uniform_at_scale_zero(w):
    """Scale 0: every query head averages the leading d_v columns of its
    sequence's rows uniformly; lse = log T."""
    inp = gi.small_wide(2, 4, 1, 10, 6, [7, 2], 8, seed=311)
    kv = gi.to_f64(inp.kv_cache, "bf16")
    got, lse = w.decode_wide(gi.to_f64(inp.q, "bf16"), kv, inp.seq_lens, 6, 0.0, return_lse=True)
    for b, T in enumerate(inp.seq_lens):
        mean = kv[b, 0, :T, :6].sum(axis=0) / T
        assert np.max(np.abs(got[b] - mean)) <= 1e-14
        assert np.max(np.abs(lse[b] - math.log(T))) <= 1e-14


def pin_rotary_columns_only_score(w):
    """The trailing (rotary) columns of a row never enter the output
    directly: with those query columns zero, changing them leaves the
    output unchanged; with nonzero rotary queries the output moves."""
    inp = gi.small_wide(1, 4, 1, 12, 8, [6], 6, seed=313)
    q, kv = gi.to_f64(inp.q, "bf16"), gi.to_f64(inp.kv_cache, "bf16")
    q0 = q.copy()
    q0[..., 8:] = 0.0
    kv2 = kv.copy()
    kv2[..., 8:] += np.arange(kv.shape[2])[None, None, :, None]   # a different shift per token
    a = w.decode_wide(q0, kv, inp.seq_lens, 8, 0.4)
    b = w.decode_wide(q0, kv2, inp.seq_lens, 8, 0.4)
    assert np.array_equal(a, b)
    c = w.decode_wide(q, kv, inp.seq_lens, 8, 0.4)
    d = w.decode_wide(q, kv2, inp.seq_lens, 8, 0.4)
    assert np.max(np.abs(c - d)) > 1e-3


def pin_empty_sequence(w):
    inp = gi.small_wide(2, 4, 2, 8, 4, [0, 3], 4, seed=317)
    out, lse = w.decode_wide(gi.to_f64(inp.q, "bf16"), gi.to_f64(inp.kv_cache, "bf16"), inp.seq_lens, 4,
                             0.5, return_lse=True)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(out[1]))


WIDE_PINS = [
    pin_absorption_equivalence,
    pin_wide_brute,
    pin_whole_row_value_is_decode,
    pin_uniform_at_scale_zero,
    pin_rotary_columns_only_score,
    pin_empty_sequence,
]
