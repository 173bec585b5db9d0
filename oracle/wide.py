"""Float64 decode in the absorbed-MLA shape: many query heads sharing one wide
cached row that serves as the key and, in its leading columns, as the value.

TEST INFRASTRUCTURE ONLY (see the package docstring): the HIP library never
imports or calls this module.

Source followed: anrans.github.io, "Attention variants: MQA, GQA, MLA",
section "MLA: multi-head latent attention".  With weight absorption the
query is projected into the latent space and scored directly against the
cached latent vectors, and the weighted sum is also taken in the latent space
(the up-projection of values moves into the output projection), so decode
attention becomes all query heads sharing one latent K that is also V, an
MQA with a very large head dimension.  The decoupled-RoPE paragraph adds a
small rotary key part, shared by all heads and cached next to the latent
vector (512 + 64 = 576 numbers per token for DeepSeek-V3).

Reading of that passage (listed in the design notes): a cached row is
[latent c (d_v columns) | rotary key (d_k - d_v columns)], the key is the
whole row and the value is its first d_v columns; the query row is
[absorbed query (d_v) | rotary query (d_k - d_v)]; the output stays in the
latent space (d_v columns).  KV heads are grouped as everywhere else: query
head h reads KV head h // (Hq / Hkv), which for the MLA shape (Hkv = 1) is
the single shared latent head.

Plain definition, whole rows, float64: no blocking, no online softmax.
"""
from __future__ import annotations

import numpy as np

from .attention import _as_f64, expand_kv_heads, group_size, softmax_average


def decode_wide(q, kv_cache, seq_lens, d_v: int, scale: float, return_lse: bool = False):
    """One decode step over a cache whose rows are both key and value.

    q [B, Hq, d_k]; kv_cache [B, Hkv, T_cap, d_k]; seq_lens [B].  Scores use
    all d_k columns; values are the first ``d_v`` columns of the same rows.
    Returns float64 out [B, Hq, d_v] (and lse [B, Hq], natural log); an empty
    sequence gives zeros and lse = -inf."""
    q = _as_f64(q)
    B, Hq, d_k = q.shape
    Hkv = kv_cache.shape[1]
    if not 0 < d_v <= d_k:
        raise ValueError(f"d_v={d_v} must be in 1..d_k={d_k}")
    g = group_size(Hq, Hkv)
    out = np.zeros((B, Hq, d_v))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        T = int(seq_lens[b])
        if T <= 0:
            continue
        rows = expand_kv_heads(_as_f64(kv_cache[b, :, :T]), g, axis=0)   # [Hq, T, d_k]
        s = scale * np.matmul(rows, q[b][:, :, None])[..., 0]             # [Hq, T]
        out[b], lse[b] = softmax_average(s, rows[..., :d_v])
    return (out, lse) if return_lse else out
