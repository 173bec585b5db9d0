"""Decode over a paged KV cache, in float64.

TEST INFRASTRUCTURE ONLY: the HIP library never imports or calls this module.

Sources (page title, then section):

* deepconcepts.dev, "Grouped-Query Attention", section "Checking it on a real
  system": paged attention is a serving-time lever on the same cache bytes
  (it stops wasting them); it changes how the cache is stored, not what
  attention computes.
* lihaoran.work, section "Check the actual deployment": GQA and
  PagedAttention act on different layers, sharing structure versus
  KV-cache organisation.
* study.greatitself.com, "Grouped-Query and Multi-Query Attention", section
  "Share keys and values without confusing query-head identity": page
  tables are storage outside the logical K/V payload.

The pages fix no page layout.  The reading used here: a pool of pages
``[num_pages, Hkv, page_size, d]`` and a block table whose entry ``[b, i]``
names the page holding tokens ``i*page_size .. (i+1)*page_size - 1`` of
sequence ``b``.  The oracle gathers each sequence's pages in table order back
into the contiguous ``[B, Hkv, T, d]`` cache and then applies the plain
decode definition unchanged.
"""
from __future__ import annotations

import numpy as np

from .attention import decode


def gather_pages(pages, block_table, seq_lens, page_size: int) -> np.ndarray:
    """Contiguous ``[B, Hkv, max_pages*page_size, d]`` cache rebuilt from the
    pool; token positions at or past ``seq_lens[b]`` are zero (never read)."""
    pages = np.asarray(pages)
    table = np.asarray(block_table)
    B, max_pages = table.shape
    _, Hkv, ps, d = pages.shape
    if ps != page_size:
        raise ValueError("page_size disagrees with the pool's page axis")
    out = np.zeros((B, Hkv, max_pages * page_size, d), dtype=pages.dtype)
    for b in range(B):
        t = int(seq_lens[b])
        for i in range(-(-t // page_size)):
            pid = int(table[b, i])
            if not 0 <= pid < pages.shape[0]:
                raise ValueError(f"block_table[{b}, {i}] = {pid} is not a page of the pool")
            n = min(page_size, t - i * page_size)
            out[b, :, i * page_size:i * page_size + n] = pages[pid, :, :n]
    return out


def decode_paged(q, k_pages, v_pages, block_table, seq_lens, page_size: int, scale: float,
                 return_lse: bool = False):
    """Decode output ``[B, Hq, d]`` over a paged cache: gather, then decode."""
    k = gather_pages(np.asarray(k_pages, dtype=np.float64), block_table, seq_lens, page_size)
    v = gather_pages(np.asarray(v_pages, dtype=np.float64), block_table, seq_lens, page_size)
    return decode(q, k, v, seq_lens, scale, return_lse=return_lse)
