"""Pins of the paged-cache oracle (oracle/paged.py).

Each pin takes the paged module so test_oracle_paged.py can also run them
against deliberately broken copies.  They check the oracle against the
contiguous oracle after an independent scatter (exact equality: the gathered
values and the float64 arithmetic are identical), against a scalar brute
force that follows the block table token by token, and against structural
facts (table order matters, one page per token)."""
import numpy as np

import gqa_inputs as gi
import oracle
from brute import brute_decode_paged


def _lists(x):
    return np.asarray(x, dtype=np.float64).tolist()


def pin_paged_brute(p):
    """Tiny case against the token-by-token brute force."""
    inp = gi.small_decode("f32", 2, 4, 2, 3, [5, 3], 6, seed=211)
    pg = gi.make_paged(inp, page_size=2, spare_pages=3, seed=5)
    scale = 0.7
    got = p.decode_paged(pg.q, pg.k_pages, pg.v_pages, pg.block_table, pg.seq_lens, 2, scale)
    ref = np.asarray(brute_decode_paged(_lists(pg.q), _lists(pg.k_pages), _lists(pg.v_pages),
                                        pg.block_table.tolist(), pg.seq_lens.tolist(), 2, scale))
    assert np.max(np.abs(got - ref)) <= 1e-12


def pin_paged_equals_contiguous(p):
    """A permuted page pool decodes exactly like the contiguous cache it was
    scattered from, for several page sizes (including a partial last page and
    a one-token sequence)."""
    inp = gi.small_decode("bf16", 3, 8, 2, 16, [37, 1, 64], 64, seed=223)
    q = gi.to_f64(inp.q, "bf16")
    ref = oracle.decode(q, gi.to_f64(inp.k_cache, "bf16"), gi.to_f64(inp.v_cache, "bf16"),
                        inp.seq_lens, 0.25)
    for ps in (4, 16, 64):
        pg = gi.make_paged(inp, page_size=ps, seed=ps)
        got = p.decode_paged(q, gi.to_f64(pg.k_pages, "bf16"), gi.to_f64(pg.v_pages, "bf16"),
                             pg.block_table, pg.seq_lens, ps, 0.25)
        assert np.array_equal(got, ref), ps


def pin_token_pages(p):
    """page_size 1 (one token per page) is the same attention."""
    inp = gi.small_decode("f32", 2, 6, 3, 8, [9, 4], 12, seed=227)
    pg = gi.make_paged(inp, page_size=1, seed=3)
    ref = oracle.decode(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, 0.3)
    got = p.decode_paged(pg.q, pg.k_pages, pg.v_pages, pg.block_table, pg.seq_lens, 1, 0.3)
    assert np.array_equal(got, ref)


def pin_gather_roundtrip(p):
    """Gathering the scattered pool returns the original tokens in order."""
    inp = gi.small_decode("f32", 2, 4, 2, 5, [11, 7], 12, seed=229)
    pg = gi.make_paged(inp, page_size=4, seed=9)
    k = p.gather_pages(pg.k_pages, pg.block_table, pg.seq_lens, 4)
    for b, t in enumerate(inp.seq_lens):
        assert np.array_equal(k[b, :, :t], inp.k_cache[b, :, :t])


def pin_table_entries_select_pages(p):
    """The table decides which pages are read: swapping two full pages of one
    sequence only reorders its tokens (attention over all of them is
    order-free, so the output agrees to rounding), while pointing an entry
    at another sequence's page changes the output."""
    inp = gi.small_decode("f32", 2, 4, 1, 8, [16, 16], 16, seed=233)
    pg = gi.make_paged(inp, page_size=4, seed=11)
    a = p.decode_paged(pg.q, pg.k_pages, pg.v_pages, pg.block_table, pg.seq_lens, 4, 0.5)
    t2 = pg.block_table.copy()
    t2[0, [0, 2]] = t2[0, [2, 0]]
    b = p.decode_paged(pg.q, pg.k_pages, pg.v_pages, t2, pg.seq_lens, 4, 0.5)
    assert np.allclose(a, b, rtol=0, atol=1e-12)
    t3 = pg.block_table.copy()
    t3[0, 1] = t3[1, 1]
    c = p.decode_paged(pg.q, pg.k_pages, pg.v_pages, t3, pg.seq_lens, 4, 0.5)
    assert not np.allclose(a[0], c[0]) and np.array_equal(a[1], c[1])


PAGED_PINS = [pin_paged_brute, pin_paged_equals_contiguous, pin_token_pages, pin_gather_roundtrip,
              pin_table_entries_select_pages]
