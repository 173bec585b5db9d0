"""Closed forms for KV-cache size and attention work.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (page title, then section):

* deepconcepts.dev, "Grouped-Query Attention": the per-token cache size is
  2 (K and V) x layers x KV heads x head dim x bytes per element, with no
  query-head term; a decode step does 4 x layers x query heads x head dim
  FLOPs per cached token, so FLOPs per cache byte equal the group size
  (section "Three numbers that people expect to move together"); the worked
  Qwen3-8B figure in section "Checking it on a real system".
* lihaoran.work, "KV-head count determines the raw cache ratio": raw bytes of
  one request are 2 x L x T x Hkv x d x b, and a ragged batch sums the actual
  lengths.
* anrans.github.io, "Attention variants: MQA, GQA, MLA": section "How big is
  the KV cache" (per-token table) and the "Exercises" concurrency estimate
  (free memory divided by the cache of one request).
"""
from __future__ import annotations

from typing import Iterable, Union


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, bytes_per_elem: int) -> int:
    """Cache bytes added by one token: 2 * L * Hkv * d * b."""
    return 2 * layers * kv_heads * head_dim * bytes_per_elem


def kv_cache_bytes(layers: int, tokens: Union[int, Iterable[int]], kv_heads: int,
                   head_dim: int, bytes_per_elem: int) -> int:
    """Raw cache bytes 2 * L * T * Hkv * d * b; for several requests of
    different lengths, T is the sum of their cached lengths."""
    total = tokens if isinstance(tokens, int) else sum(int(t) for t in tokens)
    return total * kv_bytes_per_token(layers, kv_heads, head_dim, bytes_per_elem)


def decode_attention_flops(layers: int, q_heads: int, head_dim: int,
                           tokens: Union[int, Iterable[int]]) -> int:
    """Decode attention FLOPs: 4 * L * Hq * d per cached token (a multiply and
    an add for q.k, and again for p*v, per head coordinate)."""
    total = tokens if isinstance(tokens, int) else sum(int(t) for t in tokens)
    return 4 * layers * q_heads * head_dim * total


def causal_prefill_flops(batch: int, q_heads: int, seq_len: int, head_dim: int) -> int:
    """Exact causal prefill FLOPs: row i attends i+1 keys, costing 4*d*(i+1)
    FLOPs per head (same per-key count as decode), summed over rows."""
    return 4 * batch * q_heads * head_dim * seq_len * (seq_len + 1) // 2


def max_concurrent_requests(total_bytes: float, weight_bytes: float, reserve_bytes: float,
                            kv_per_token: int, tokens_per_request: int) -> int:
    """Requests whose caches fit in the memory left after weights and a
    reserve (anrans.github.io, "Exercises", question 1)."""
    return int((total_bytes - weight_bytes - reserve_bytes) // (kv_per_token * tokens_per_request))
