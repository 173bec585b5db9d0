"""Float64 gradients of causal GQA prefill, by repeating K/V and summing back.

TEST INFRASTRUCTURE ONLY (see the package docstring): the HIP library never
imports or calls this module.

Source followed: study.greatitself.com, "Grouped-Query and Multi-Query
Attention", section "Share keys and values without confusing query-head
identity", its paragraph on training: each shared KV head receives the sum of
the gradients of all query heads in its group.  The reference form the page
allows expands K/V per query head and adds the per-head gradients back onto
each shared KV head; this module does that, writing the chain rule out per
query head instead of leaving it to an autodiff system.

For one query head h with repeated K_h = K[h // g], V_h = V[h // g] and the
loss gradient dO_h (the caller's upstream gradient of the output), the
forward of the causal prefill oracle is

    S = scale * Q_h K_h^T   with S[i, t] = -inf for keys t > i,
    P = softmax over each row of S,        O_h = P V_h,

and its reverse pass through those three steps is

    dV_h = P^T dO_h                              (O = P V, with respect to V)
    dP   = dO_h V_h^T                            (O = P V, with respect to P)
    dS   = P * (dP - rowsum(P * dP))             (row softmax Jacobian)
    dQ_h = scale * dS K_h                        (S = scale Q K^T)
    dK_h = scale * dS^T Q_h

The repeat copies KV head j to query heads j*g .. j*g+g-1, so its adjoint is
the sum over those g heads: dK[j] = sum of dK_h, dV[j] = sum of dV_h.

Masked entries have P = 0 and so contribute nothing.  Whole rows, whole
matrices and float64 throughout: no tiling, no recomputation from a stored
log-sum-exp, no fused rowsum(dO * O).
"""
from __future__ import annotations

import numpy as np

from .attention import _as_f64, _causal_scores, expand_kv_heads, group_size


def reduce_kv_heads(x: np.ndarray, g: int, axis: int) -> np.ndarray:
    """Adjoint of ``expand_kv_heads``: sum each run of g consecutive entries
    of the head axis back onto the KV head they were copied from."""
    x = np.moveaxis(np.asarray(x), axis, 0)
    hq = x.shape[0]
    out = x.reshape((hq // g, g) + x.shape[1:]).sum(axis=1)
    return np.moveaxis(out, 0, axis)


def softmax_rows(scores: np.ndarray) -> np.ndarray:
    """Row softmax of ``scores`` [N, T] with -inf entries mapped to 0 (every
    causal row has key 0 unmasked, so each row has a finite maximum)."""
    m = np.max(scores, axis=-1, keepdims=True)
    w = np.exp(scores - m)
    return w / np.sum(w, axis=-1, keepdims=True)


def head_backward(q_h, k_h, v_h, do_h, scale: float):
    """Gradients of one query head's causal attention.

    q_h, do_h [N, d] (this head's queries and upstream output gradient);
    k_h, v_h [N, d] (the K/V rows this head reads).  Returns (dq_h, dk_h,
    dv_h), each [N, d]: the contributions of this head alone."""
    n = q_h.shape[0]
    s = _causal_scores(q_h, k_h, np.arange(n), scale)
    p = softmax_rows(s)
    dv_h = p.T @ do_h
    dp = do_h @ v_h.T
    ds = p * (dp - np.sum(p * dp, axis=-1, keepdims=True))
    dq_h = scale * (ds @ k_h)
    dk_h = scale * (ds.T @ q_h)
    return dq_h, dk_h, dv_h


def prefill_causal_backward(q, k, v, dout, scale: float):
    """Gradients of causal GQA prefill with respect to q, k and v.

    q, dout [B, Hq, N, d]; k, v [B, Hkv, N, d].  Returns float64
    (dq [B, Hq, N, d], dk [B, Hkv, N, d], dv [B, Hkv, N, d]) of the loss whose
    gradient with respect to the attention output is ``dout``."""
    q, k, v, do = (_as_f64(x) for x in (q, k, v, dout))
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    g = group_size(Hq, Hkv)
    dq = np.zeros((B, Hq, N, d))
    dk = np.zeros((B, Hkv, N, d))
    dv = np.zeros((B, Hkv, N, d))
    if N == 0:
        return dq, dk, dv
    for b in range(B):
        k_exp = expand_kv_heads(k[b], g, axis=0)   # [Hq, N, d]
        v_exp = expand_kv_heads(v[b], g, axis=0)
        dk_exp = np.empty((Hq, N, d))
        dv_exp = np.empty((Hq, N, d))
        for h in range(Hq):
            dq[b, h], dk_exp[h], dv_exp[h] = head_backward(q[b, h], k_exp[h], v_exp[h], do[b, h], scale)
        dk[b] = reduce_kv_heads(dk_exp, g, axis=0)
        dv[b] = reduce_kv_heads(dv_exp, g, axis=0)
    return dq, dk, dv


def prefill_causal_backward_group(q_b, k_b, v_b, dout_b, kvh: int, scale: float):
    """The gradients that involve one KV head of one sequence: dq of its g
    query heads and dk, dv of the KV head itself.

    q_b, dout_b [Hq, N, d]; k_b, v_b [Hkv, N, d].  Returns (dq [g, N, d],
    dk [N, d], dv [N, d]) equal to the matching slices of
    ``prefill_causal_backward`` (the group's heads read nothing else), for
    checks on workloads too large to differentiate whole."""
    Hq = q_b.shape[0]
    Hkv = k_b.shape[0]
    g = group_size(Hq, Hkv)
    heads = slice(kvh * g, (kvh + 1) * g)
    dq, dk, dv = prefill_causal_backward(np.asarray(q_b)[None, heads], np.asarray(k_b)[None, kvh:kvh + 1],
                                         np.asarray(v_b)[None, kvh:kvh + 1],
                                         np.asarray(dout_b)[None, heads], scale)
    return dq[0], dk[0, 0], dv[0, 0]
