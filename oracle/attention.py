"""Plain float64 grouped-query attention, with K/V explicitly repeated.

TEST INFRASTRUCTURE ONLY (see the package docstring): the HIP library never
imports or calls this module.

Sources followed (page title, then section):

* study.greatitself.com, "Grouped-Query and Multi-Query Attention", section
  "Share keys and values without confusing query-head identity": Hq must be
  a multiple of Hkv; consecutive blocks of Hq/Hkv query heads share one KV
  head; each query head keeps its own distribution and output; a reference
  may repeat K and V along the query-head axis.
* lihaoran.work, "Shared KV can still produce different outputs" (the
  teaching script): the mapping h // (Hq/Hkv), scores divided by sqrt(d),
  max-subtracted exponentials, weighted average of the values.
* anrans.github.io, "Attention variants: MQA, GQA, MLA", section "Kernels do
  not need to copy the KV heads": the repeat_interleave form, the
  lower-triangular causal mask, softmax over the key axis, then times V.

Readings where the pages are silent (each listed in the design notes):

* decode attends to all ``seq_lens[b]`` cached tokens, with no mask;
* an empty softmax (``seq_lens[b] == 0``) yields an all-zero output and a
  log-sum-exp of -inf;
* the scale is a caller argument (the workloads pass 1/sqrt(d)).

No blocking, online softmax or split is used here: each output row is the
whole-row softmax of its scores, computed in one pass in float64.
"""
from __future__ import annotations

import numpy as np


def group_size(num_q_heads: int, num_kv_heads: int) -> int:
    """Query heads per KV head, g = Hq / Hkv.

    The grouping is only defined when Hkv >= 1 divides Hq (study.greatitself.com,
    "Share keys and values without confusing query-head identity"; the
    divisibility assert of the lihaoran.work teaching script)."""
    if num_kv_heads < 1 or num_q_heads < 1 or num_q_heads % num_kv_heads != 0:
        raise ValueError(f"Hq={num_q_heads} is not a positive multiple of Hkv={num_kv_heads}")
    return num_q_heads // num_kv_heads


def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head ``h``: h // (Hq/Hkv) (lihaoran.work teaching
    script; anrans.github.io self-test answer 2)."""
    return h // group_size(num_q_heads, num_kv_heads)


def head_mapping(num_q_heads: int, num_kv_heads: int) -> list:
    """The KV head of every query head, in query-head order."""
    return [kv_head_of(h, num_q_heads, num_kv_heads) for h in range(num_q_heads)]


def expand_kv_heads(x: np.ndarray, g: int, axis: int) -> np.ndarray:
    """Materialised per-query-head copy of K or V (repeat_interleave order).

    Element j of the head axis is copied to positions j*g .. j*g+g-1, which is
    the consecutive grouping (anrans.github.io, "Kernels do not need to copy
    the KV heads", version 1).  A tiled copy (j at j, j+Hkv, ...) would be the
    wrong, strided grouping."""
    return np.repeat(x, g, axis=axis)


def softmax_average(scores: np.ndarray, values: np.ndarray):
    """Softmax over the last axis of ``scores`` [..., T], applied to
    ``values`` [..., T, d].  Returns (output [..., d], lse [...]).

    Max-subtracted exponentials as in the lihaoran.work teaching script; masked
    entries are -inf and contribute exp(-inf) = 0.  ``lse`` is the natural
    log-sum-exp of the scores."""
    m = np.max(scores, axis=-1, keepdims=True)
    w = np.exp(scores - m)
    den = np.sum(w, axis=-1)
    num = np.matmul(w[..., None, :], values)[..., 0, :]
    return num / den[..., None], m[..., 0] + np.log(den)


def _as_f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def decode(q, k_cache, v_cache, seq_lens, scale: float, return_lse: bool = False):
    """One decode step: every query head attends to its sequence's cache.

    q [B, Hq, d]; k_cache, v_cache [B, Hkv, T_cap, d]; seq_lens [B].
    Returns float64 out [B, Hq, d] (and lse [B, Hq], natural log).

    out[b, h] = sum_t softmax_t(scale * q[b,h] . K_exp[b,h,t]) V_exp[b,h,t]
    over t < seq_lens[b], with K_exp/V_exp the head-repeated caches."""
    q = _as_f64(q)
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    g = group_size(Hq, Hkv)
    out = np.zeros((B, Hq, d))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        T = int(seq_lens[b])
        if T <= 0:
            continue
        k_exp = expand_kv_heads(_as_f64(k_cache[b, :, :T]), g, axis=0)   # [Hq, T, d]
        v_exp = expand_kv_heads(_as_f64(v_cache[b, :, :T]), g, axis=0)
        s = scale * np.matmul(k_exp, q[b][:, :, None])[..., 0]          # [Hq, T]
        out[b], lse[b] = softmax_average(s, v_exp)
    return (out, lse) if return_lse else out


def decode_one(q_bh, k_cache_b, v_cache_b, seq_len: int, h: int, num_q_heads: int,
               scale: float):
    """Decode output of one (sequence, query head) pair, for sampled checks on
    workloads too large to expand whole.

    q_bh [d]; k_cache_b, v_cache_b [Hkv, T_cap, d].  The KV head is chosen
    by the same repeat applied to the head indices, then the plain softmax
    average over the first ``seq_len`` tokens.  Returns (out [d], lse)."""
    Hkv = k_cache_b.shape[0]
    g = group_size(num_q_heads, Hkv)
    src = expand_kv_heads(np.arange(Hkv), g, axis=0)[h]
    T = int(seq_len)
    if T <= 0:
        return np.zeros(k_cache_b.shape[-1]), -np.inf
    k = _as_f64(k_cache_b[src, :T])
    v = _as_f64(v_cache_b[src, :T])
    s = scale * (k @ _as_f64(q_bh))
    out, lse = softmax_average(s, v)
    return out, float(lse)


def _causal_scores(q_rows, k, rows, scale):
    """scale * q_rows . k^T with key j > query position i set to -inf
    (lower-triangular mask, anrans.github.io version 1)."""
    s = scale * (q_rows @ k.T)
    j = np.arange(k.shape[0])[None, :]
    return np.where(j <= np.asarray(rows)[:, None], s, -np.inf)


def prefill_causal(q, k, v, scale: float, return_lse: bool = False):
    """Causal self-attention over a whole prompt.

    q [B, Hq, N, d]; k, v [B, Hkv, N, d].  Row i of head h attends to keys
    0..i of KV head h // g.  Returns float64 out [B, Hq, N, d] (and lse
    [B, Hq, N])."""
    q = _as_f64(q)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    g = group_size(Hq, Hkv)
    out = np.empty((B, Hq, N, d))
    lse = np.empty((B, Hq, N))
    rows = np.arange(N)
    for b in range(B):
        k_exp = expand_kv_heads(_as_f64(k[b]), g, axis=0)   # [Hq, N, d]
        v_exp = expand_kv_heads(_as_f64(v[b]), g, axis=0)
        for h in range(Hq):
            s = _causal_scores(q[b, h], k_exp[h], rows, scale)
            out[b, h], lse[b, h] = softmax_average(s, v_exp[h])
    return (out, lse) if return_lse else out


def prefill_causal_rows(q_bh_rows, k_b, v_b, rows, h: int, num_q_heads: int, scale: float):
    """Selected rows of one (sequence, query head) of causal prefill.

    q_bh_rows [R, d] are the queries at positions ``rows``; k_b, v_b
    [Hkv, N, d].  Returns (out [R, d], lse [R])."""
    Hkv = k_b.shape[0]
    g = group_size(num_q_heads, Hkv)
    src = expand_kv_heads(np.arange(Hkv), g, axis=0)[h]
    rows = np.asarray(rows)
    last = int(rows.max()) + 1
    k = _as_f64(k_b[src, :last])
    v = _as_f64(v_b[src, :last])
    s = _causal_scores(_as_f64(q_bh_rows), k, rows, scale)
    return softmax_average(s, v)
