"""Pins of the prefill-gradient oracle (oracle/backward.py).

Each pin takes the backward module so test_oracle_backward.py can also run
them against deliberately broken copies.  None of them re-derives the
gradient formulas: they check the oracle against

* central finite differences of the (separately pinned) forward oracle,
* torch's own autograd through its GQA attention (CPU, float64),
* closed forms: uniform attention at scale 0, the first row, the sums of
  the key and value gradients over tokens, and two inner-product identities,
* the group structure: GQA gradients equal MHA gradients over explicitly
  repeated K/V, summed over each group, and the repeat and the sum are
  adjoint."""
import numpy as np
import torch

import oracle


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _case(seed, B, Hq, Hkv, N, d):
    return (_rand(seed, B, Hq, N, d), _rand(seed + 1, B, Hkv, N, d),
            _rand(seed + 2, B, Hkv, N, d), _rand(seed + 3, B, Hq, N, d))


def pin_finite_differences(bw):
    """Every gradient entry against a central difference of
    L = sum(dout * forward(q, k, v)), the forward being the pinned oracle."""
    for seed, shape, scale in ((11, (1, 4, 2, 5, 3), 0.6), (21, (1, 3, 1, 4, 2), 1.1),
                               (31, (2, 2, 2, 3, 2), -0.4)):
        q, k, v, do = _case(seed, *shape)
        grads = bw.prefill_causal_backward(q, k, v, do, scale)

        def loss(q_, k_, v_):
            return float(np.sum(do * oracle.prefill_causal(q_, k_, v_, scale)))

        eps = 1e-6
        for which, g in enumerate(grads):
            args = [q, k, v]
            base = args[which]
            for idx in np.ndindex(base.shape):
                plus, minus = base.copy(), base.copy()
                plus[idx] += eps
                minus[idx] -= eps
                a = list(args)
                a[which] = plus
                lp = loss(*a)
                a[which] = minus
                lm = loss(*a)
                fd = (lp - lm) / (2 * eps)
                assert abs(g[idx] - fd) <= 1e-6 * (1 + abs(fd)), (seed, which, idx, g[idx], fd)


def pin_torch_autograd(bw):
    """torch's causal GQA attention (enable_gqa, math path, CPU float64) and
    its autograd, on shapes with several groups, a group of 3 and MQA."""
    for seed, shape, scale in ((41, (2, 8, 2, 37, 16), 0.25), (51, (1, 6, 2, 19, 8), 0.5),
                               (61, (1, 5, 1, 23, 4), 0.9)):
        q, k, v, do = _case(seed, *shape)
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale,
                                                               enable_gqa=True)
        out.backward(torch.tensor(do))
        got = bw.prefill_causal_backward(q, k, v, do, scale)
        for g, t in zip(got, (tq, tk, tv)):
            ref = t.grad.numpy()
            assert g.shape == ref.shape
            assert np.max(np.abs(g - ref)) <= 1e-10 * (1 + np.max(np.abs(ref))), seed


def pin_uniform_attention(bw):
    """At scale 0 every row averages its keys uniformly: dq = dk = 0 and
    dv[j, t] = sum over the group's heads h and rows i >= t of dout[h, i] / (i + 1)."""
    B, Hq, Hkv, N, d = 1, 6, 2, 7, 3
    q, k, v, do = _case(71, B, Hq, Hkv, N, d)
    dq, dk, dv = bw.prefill_causal_backward(q, k, v, do, 0.0)
    assert np.all(dq == 0) and np.all(dk == 0)
    g = Hq // Hkv
    for j in range(Hkv):
        for t in range(N):
            ref = sum(do[0, h, i] / (i + 1) for h in range(j * g, (j + 1) * g) for i in range(t, N))
            assert np.max(np.abs(dv[0, j, t] - ref)) <= 1e-12


def pin_first_row(bw):
    """Row 0 sees only key 0, so its softmax is constant: dq of row 0 is
    exactly zero, and key/value 0 are the only ones it touches."""
    q, k, v, do = _case(81, 1, 4, 2, 6, 5)
    dq, _, _ = bw.prefill_causal_backward(q, k, v, do, 0.7)
    assert np.all(dq[:, :, 0] == 0)
    assert np.all(np.abs(dq[:, :, 1:]).sum(axis=-1) > 0)
    # The last key is seen only by the last row: its value gradient is the
    # last row's dout weighted by that row's probability of the last key,
    # summed over the group.
    _, _, dv = bw.prefill_causal_backward(q, k, v, do, 0.0)
    assert np.allclose(dv[0, 0, -1], (do[0, 0, -1] + do[0, 1, -1]) / 6, rtol=0, atol=1e-14)


def pin_token_sums(bw):
    """Shifting every key by one vector leaves each row's softmax unchanged,
    so the key gradient sums to zero over tokens; rows of P sum to one, so the
    value gradient sums to the group's dout summed over rows."""
    B, Hq, Hkv, N, d = 2, 8, 2, 11, 4
    q, k, v, do = _case(91, B, Hq, Hkv, N, d)
    _, dk, dv = bw.prefill_causal_backward(q, k, v, do, 0.45)
    g = Hq // Hkv
    for b in range(B):
        for j in range(Hkv):
            assert np.max(np.abs(dk[b, j].sum(axis=0))) <= 1e-12
            ref = sum(do[b, h].sum(axis=0) for h in range(j * g, (j + 1) * g))
            assert np.max(np.abs(dv[b, j].sum(axis=0) - ref)) <= 1e-12


def pin_inner_products(bw):
    """Scaling all queries or all keys of a group by (1 + e) moves the
    scores alike, so sum_h <q_h, dq_h> = <k, dk>; and sum_t <v_t, dv_t> =
    sum_h <out_h, dout_h> since out is linear in v."""
    B, Hq, Hkv, N, d = 1, 6, 3, 9, 5
    q, k, v, do = _case(101, B, Hq, Hkv, N, d)
    dq, dk, dv = bw.prefill_causal_backward(q, k, v, do, 0.8)
    out = oracle.prefill_causal(q, k, v, 0.8)
    g = Hq // Hkv
    for j in range(Hkv):
        heads = range(j * g, (j + 1) * g)
        qq = sum(np.sum(q[0, h] * dq[0, h]) for h in heads)
        assert abs(qq - np.sum(k[0, j] * dk[0, j])) <= 1e-12 * (1 + abs(qq))
        oo = sum(np.sum(out[0, h] * do[0, h]) for h in heads)
        assert abs(oo - np.sum(v[0, j] * dv[0, j])) <= 1e-12 * (1 + abs(oo))


def pin_group_sum_equals_mha(bw):
    """GQA gradients equal MHA gradients over K/V repeated per query head
    (by an index loop here), with dk, dv summed over each group."""
    B, Hq, Hkv, N, d = 2, 8, 2, 13, 6
    q, k, v, do = _case(111, B, Hq, Hkv, N, d)
    g = Hq // Hkv
    k_rep = np.stack([k[:, h // g] for h in range(Hq)], axis=1)
    v_rep = np.stack([v[:, h // g] for h in range(Hq)], axis=1)
    dq_m, dk_m, dv_m = bw.prefill_causal_backward(q, k_rep, v_rep, do, 0.3)
    dq, dk, dv = bw.prefill_causal_backward(q, k, v, do, 0.3)
    assert np.max(np.abs(dq - dq_m)) <= 1e-12
    for j in range(Hkv):
        ref_k = sum(dk_m[:, h] for h in range(Hq) if h // g == j)
        ref_v = sum(dv_m[:, h] for h in range(Hq) if h // g == j)
        assert np.max(np.abs(dk[:, j] - ref_k)) <= 1e-12
        assert np.max(np.abs(dv[:, j] - ref_v)) <= 1e-12


def pin_group_slice(bw):
    """The one-KV-head helper returns the matching slices of the full result."""
    B, Hq, Hkv, N, d = 2, 8, 4, 10, 3
    q, k, v, do = _case(121, B, Hq, Hkv, N, d)
    dq, dk, dv = bw.prefill_causal_backward(q, k, v, do, 0.5)
    for b, j in ((0, 0), (1, 3), (1, 2)):
        gq, gk, gv = bw.prefill_causal_backward_group(q[b], k[b], v[b], do[b], j, 0.5)
        assert np.array_equal(gq, dq[b, 2 * j:2 * j + 2])
        assert np.array_equal(gk, dk[b, j]) and np.array_equal(gv, dv[b, j])


def pin_repeat_sum_adjoint(bw):
    """<repeat(x), y> = <x, sum_back(y)> for the head repeat and its adjoint,
    where repeat is the forward oracle's own head expansion."""
    x = _rand(131, 3, 5, 2)
    y = _rand(132, 12, 5, 2)
    lhs = np.sum(oracle.expand_kv_heads(x, 4, axis=0) * y)
    rhs = np.sum(x * bw.reduce_kv_heads(y, 4, axis=0))
    assert abs(lhs - rhs) <= 1e-12
    x1 = _rand(133, 2, 3, 4)
    y1 = _rand(134, 2, 6, 4)
    lhs1 = np.sum(oracle.expand_kv_heads(x1, 2, axis=1) * y1)
    assert abs(lhs1 - np.sum(x1 * bw.reduce_kv_heads(y1, 2, axis=1))) <= 1e-12


BACKWARD_PINS = [
    pin_finite_differences,
    pin_torch_autograd,
    pin_uniform_attention,
    pin_first_row,
    pin_token_sums,
    pin_inner_products,
    pin_group_sum_equals_mha,
    pin_group_slice,
    pin_repeat_sum_adjoint,
]
