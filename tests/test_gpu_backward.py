"""GPU causal prefill backward (bf16 MFMA kernels through the C ABI) against
the float64 gradient oracle.

The GPU forward supplies out and lse, as in training; the oracle recomputes
everything from q, k, v and dout.  Tolerance: max |gpu - oracle| over a
tensor <= TOL_REL * max(1, max |oracle| of that tensor) (the floor covers
gradients that are exactly zero, such as dq and dk of a one-token prompt,
where the kernels leave float32 rounding noise).  The kernels round P and dS
to bf16 before the products that consume them (2^-9 relative each), which in
a float64 simulation of exactly that rounding gives at most 2.2e-3 of
max |oracle| on these shapes and on N = 2048 and 4096; TOL_REL leaves a
4.5x margin for the forward's own rounding in out and lse."""
import zlib

import numpy as np
import pytest
import torch

import gqa_inputs as gi
import grouped_query_attention_gqa_amd as gqa
import oracle
from gpu_util import dev, need_gpu, say

pytestmark = pytest.mark.gpu

TOL_REL = 1e-2


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite GPU gradient"
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1.0))


def run_backward(p, dout_bits, scale=None):
    scale = p.cfg.scale if scale is None else scale
    q, k, v, do = dev(p.q, "bf16"), dev(p.k, "bf16"), dev(p.v, "bf16"), dev(dout_bits, "bf16")
    out, lse = gqa.gqa_prefill_causal(q, k, v, scale=scale, return_lse=True)
    dq, dk, dv = gqa.gqa_prefill_causal_backward(q, k, v, out, lse, do, scale=scale)
    torch.cuda.synchronize()
    return dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()


def oracle_grads(p, dout_bits, scale=None):
    scale = p.cfg.scale if scale is None else scale
    return oracle.prefill_causal_backward(gi.to_f64(p.q, "bf16"), gi.to_f64(p.k, "bf16"),
                                          gi.to_f64(p.v, "bf16"), gi.to_f64(dout_bits, "bf16"), scale)


SMALL = [
    # B, Hq, Hkv, N, d
    (1, 8, 2, 300, 128),     # group 4, ragged tail
    (2, 8, 2, 64, 64),       # d = 64, one key workgroup
    (1, 4, 4, 130, 128),     # MHA endpoint
    (1, 6, 2, 77, 128),      # group 3: one head per dq workgroup
    (1, 16, 1, 200, 128),    # MQA, group 16
    (1, 4, 2, 1, 128),       # a single token
    (1, 8, 4, 33, 64),       # group 2
    (1, 8, 2, 515, 128),     # five key workgroups, ragged last
    (2, 4, 1, 640, 64),      # MQA-style group 4, d = 64, several key workgroups
    (1, 3, 3, 389, 128),     # MHA, 128 positions per dq tile
    (1, 32, 8, 300, 128),    # 8 units: the per-XCD grouping of the prefill-4k launch
    (2, 16, 8, 200, 64),     # 16 units, d = 64
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}-{}on{}-N{}-d{}".format(*c))
def test_small_backward_parity(case):
    need_gpu()
    B, Hq, Hkv, N, d = case
    p = gi.small_prefill(B, Hq, Hkv, N, d, seed=zlib.crc32(repr(case).encode()) % 100000)
    do = gi.make_dout(p.cfg)
    say("backward small", case)
    got = run_backward(p, do)
    ref = oracle_grads(p, do)
    errs = [rel_err(a, r) for a, r in zip(got, ref)]
    say("rel err dq dk dv", errs)
    assert max(errs) <= TOL_REL
    # row 0 sees only key 0, so its softmax cannot move: dq of row 0 is
    # float32 rounding noise of P = exp(s - lse) ~ 1 against a sizeable rest
    assert np.max(np.abs(got[0][:, :, 0])) <= 1e-5 * max(np.max(np.abs(got[0])), 1.0)


def test_group_sum_matches_repeated_heads():
    """GQA gradients equal those of MHA over K/V repeated per query head
    (repeated on the host), with dk/dv summed over each group: dq
    bit-identical, dk/dv up to float32 summation order."""
    need_gpu()
    B, Hq, Hkv, N, d = 1, 8, 2, 333, 128
    p = gi.small_prefill(B, Hq, Hkv, N, d, seed=77)
    do = gi.make_dout(p.cfg)
    dq, dk, dv = run_backward(p, do)
    g = Hq // Hkv
    rep = gi.small_prefill(B, Hq, Hq, N, d, seed=77)
    rep.q[:] = p.q
    rep.k[:] = np.stack([p.k[:, h // g] for h in range(Hq)], axis=1)
    rep.v[:] = np.stack([p.v[:, h // g] for h in range(Hq)], axis=1)
    dq_m, dk_m, dv_m = run_backward(rep, do)
    assert np.array_equal(dq, dq_m)
    for j in range(Hkv):
        sk = dk_m[:, j * g:(j + 1) * g].astype(np.float64).sum(axis=1)
        sv = dv_m[:, j * g:(j + 1) * g].astype(np.float64).sum(axis=1)
        assert np.max(np.abs(dk[:, j] - sk)) <= 1e-5 * np.max(np.abs(sk))
        assert np.max(np.abs(dv[:, j] - sv)) <= 1e-5 * np.max(np.abs(sv))


def test_backward_deterministic():
    need_gpu()
    p = gi.small_prefill(1, 8, 2, 700, 128, seed=91)
    do = gi.make_dout(p.cfg)
    a = run_backward(p, do)
    b = run_backward(p, do)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("scale", [0.0, -0.07], ids=["zero", "negative"])
def test_backward_nonpositive_scale(scale):
    need_gpu()
    p = gi.small_prefill(1, 8, 2, 200, 128, seed=53)
    do = gi.make_dout(p.cfg)
    got = run_backward(p, do, scale)
    ref = oracle_grads(p, do, scale)
    if scale == 0.0:
        assert np.all(got[0] == 0) and np.all(got[1] == 0)
        errs = [rel_err(got[2], ref[2])]
    else:
        errs = [rel_err(a, r) for a, r in zip(got, ref)]
    say("scale", scale, "rel err", errs)
    assert max(errs) <= TOL_REL


@pytest.mark.parametrize("quarter", range(4))
def test_prefill_4k_backward_full_size(quarter):
    """The full prefill-4k workload (B=2, Hq=32, Hkv=8, N=4096, d=128) in the
    bench's launch configuration; the oracle differentiates every KV-head
    group (all 4096 rows of its 4 query heads, and the group's dk and dv),
    four of the sixteen (sequence, KV head) groups per test."""
    need_gpu()
    cfg = gi.CONFIGS["prefill-4k"]
    p = gi.make_prefill(cfg)
    do = gi.make_dout(cfg)
    say("prefill-4k backward", gi.describe(cfg), "quarter", quarter)
    dq, dk, dv = run_backward(p, do)
    for x in (dq, dk, dv):
        assert np.all(np.isfinite(x))
    g = cfg.num_q_heads // cfg.num_kv_heads
    groups = [(b, j) for b in range(cfg.batch) for j in range(cfg.num_kv_heads)]
    per = len(groups) // 4
    worst = 0.0
    for b, j in groups[quarter * per:(quarter + 1) * per]:
        rq, rk, rv = oracle.prefill_causal_backward_group(
            gi.to_f64(p.q[b], "bf16"), gi.to_f64(p.k[b], "bf16"), gi.to_f64(p.v[b], "bf16"),
            gi.to_f64(do[b], "bf16"), j, cfg.scale)
        errs = [rel_err(dq[b, j * g:(j + 1) * g], rq), rel_err(dk[b, j], rk), rel_err(dv[b, j], rv)]
        say("group", (b, j), "rel err dq dk dv", errs)
        worst = max(worst, *errs)
    assert worst <= TOL_REL
