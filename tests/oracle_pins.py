"""Pins of the float64 oracle, written as functions of the oracle module.

Each pin checks the oracle against something other than itself: values the
source pages print, closed forms, exact special cases, an independent
grouped-rows formulation, or the scalar brute force in ``brute.py``.  The pins
take the attention module as an argument so that test_oracle_mutants.py can
run them against deliberately broken copies and show each copy is caught.
"""
import json
import math
import os

import numpy as np

from brute import brute_decode, brute_prefill

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


# -- head mapping -------------------------------------------------------------

def pin_mapping_examples(o):
    """8 on 2 and 6 on 2, as printed (lihaoran.work teaching script;
    study.greatitself.com six-on-two example)."""
    for ex in golden("head_mapping_examples.json")["examples"]:
        assert o.head_mapping(ex["num_q_heads"], ex["num_kv_heads"]) == ex["mapping"], ex


def pin_mapping_endpoints(o):
    """MHA (Hkv = Hq) maps every head to itself; MQA (Hkv = 1) maps every head
    to KV head 0 (study.greatitself.com endpoints), including the prime
    71-on-1 case (deepconcepts.dev, Falcon-7B)."""
    assert o.head_mapping(12, 12) == list(range(12))
    assert o.head_mapping(71, 1) == [0] * 71
    assert o.head_mapping(32, 8) == [h // 4 for h in range(32)]
    assert o.head_mapping(16, 1) == [0] * 16


def pin_rejects_irregular_grouping(o):
    """Hq must be a positive multiple of Hkv >= 1 (study.greatitself.com;
    the divisibility assert of the lihaoran.work teaching script)."""
    for hq, hkv in [(6, 4), (8, 0), (8, 3)]:
        try:
            o.group_size(hq, hkv)
        except ValueError:
            continue
        raise AssertionError(f"grouping {hq} on {hkv} accepted")


def pin_expand_is_consecutive(o):
    """The repeated K holds KV head j at query heads j*g .. j*g+g-1."""
    k = _rng(1).standard_normal((2, 3, 5, 4))
    e = o.expand_kv_heads(k, 4, axis=1)
    assert e.shape == (2, 12, 5, 4)
    for h in range(12):
        assert np.array_equal(e[:, h], k[:, h // 4])


# -- page worked examples -----------------------------------------------------

def _two_query_inputs():
    g = golden("two_queries_shared_kv.json")
    q = np.array([g["queries"]], dtype=np.float64)                  # [1, 2, 2]
    k = np.array([[g["keys"]]], dtype=np.float64)                   # [1, 1, 2, 2]
    vals = g["values"]
    v = np.array([[[[vals[0], 0.0], [vals[1], 0.0]]]])              # value as a 2-vector
    return q, k, v, np.array([2]), 1.0 / math.sqrt(2.0)


def pin_two_queries_closed_form(o):
    """Two queries over the same two keys/values give different outputs
    (lihaoran.work): a=(10+20w)/(1+w), b=(10w+20)/(1+w), w=e^(-1/sqrt 2)."""
    q, k, v, lens, scale = _two_query_inputs()
    out, lse = o.decode(q, k, v, lens, scale, return_lse=True)
    w = math.exp(-1.0 / math.sqrt(2.0))
    a = (10.0 + 20.0 * w) / (1.0 + w)
    b = (10.0 * w + 20.0) / (1.0 + w)
    assert abs(out[0, 0, 0] - a) < 1e-12 and abs(out[0, 1, 0] - b) < 1e-12
    assert out[0, 0, 1] == 0.0 and out[0, 1, 1] == 0.0
    assert not math.isclose(out[0, 0, 0], out[0, 1, 0])
    assert abs(out[0, 0, 0] + out[0, 1, 0] - 30.0) < 1e-12
    s1 = 1.0 / math.sqrt(2.0)
    assert abs(lse[0, 0] - math.log(math.exp(s1) + 1.0)) < 1e-12


def grouped_rows_reference(q, k, v, scale):
    """The no-copy form (anrans.github.io, version 2): a group's query heads
    are stacked as extra query rows [B, Hkv, g*T, d] against the shared K/V,
    causal mask broadcast over the group.  Written independently of the oracle."""
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    qg = q.reshape(B, Hkv, g * T, d)
    s = (qg @ np.swapaxes(k, -1, -2)) * scale                        # [B, Hkv, g*T, T]
    s = s.reshape(B, Hkv, g, T, T)
    keep = np.tril(np.ones((T, T), dtype=bool))
    s = np.where(keep, s, -np.inf)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    out = p.reshape(B, Hkv, g * T, T) @ v
    return out.reshape(B, Hq, T, d)


def pin_grouped_rows_equivalence(o):
    """Repeat form (the oracle) equals the grouped-rows form on the page's
    causal 12-on-3 shape (the page asserts agreement to 1e-5; float64 here
    gives 1e-12)."""
    ex = golden("grouped_rows_example.json")
    r = _rng(ex["numpy_seed"])
    B, T, Hq, Hkv, d = ex["batch"], ex["seq_len"], ex["num_q_heads"], ex["num_kv_heads"], ex["head_dim"]
    q = r.standard_normal((B, Hq, T, d))
    k = r.standard_normal((B, Hkv, T, d))
    v = r.standard_normal((B, Hkv, T, d))
    scale = 1.0 / math.sqrt(d)
    got = o.prefill_causal(q, k, v, scale)
    ref = grouped_rows_reference(q, k, v, scale)
    assert np.max(np.abs(got - ref)) < 1e-12
    assert np.max(np.abs(got - ref)) <= ex["page_tolerance"]


# -- brute force --------------------------------------------------------------

def _lists(x):
    return x.tolist()


def pin_brute_decode(o):
    """Decode matches the scalar brute force: the tiny fp32 workload's shape
    (8 on 2, d=64, 256 tokens), 6 on 2 with ragged lengths, and 71 on 1."""
    cases = [((1, 8, 2, 64), [256], 256, 11),
             ((3, 6, 2, 8), [5, 1, 7], 7, 12),
             ((1, 71, 1, 4), [5], 6, 13)]
    for (B, Hq, Hkv, d), lens, tcap, seed in cases:
        r = _rng(seed)
        q = r.standard_normal((B, Hq, d))
        k = r.standard_normal((B, Hkv, tcap, d))
        v = r.standard_normal((B, Hkv, tcap, d))
        scale = 1.0 / math.sqrt(d)
        got = o.decode(q, k, v, np.array(lens), scale)
        ref = np.array(brute_decode(_lists(q), _lists(k), _lists(v), lens, scale))
        assert np.max(np.abs(got - ref)) < 1e-12, (B, Hq, Hkv, d)


def pin_brute_prefill(o):
    """Causal prefill matches the scalar brute force on 12 on 3 (T=9, d=16)
    and 4 on 1 (T=6, d=8)."""
    for (B, Hq, Hkv, T, d), seed in [((2, 12, 3, 9, 16), 21), ((1, 4, 1, 6, 8), 22)]:
        r = _rng(seed)
        q = r.standard_normal((B, Hq, T, d))
        k = r.standard_normal((B, Hkv, T, d))
        v = r.standard_normal((B, Hkv, T, d))
        scale = 1.0 / math.sqrt(d)
        got = o.prefill_causal(q, k, v, scale)
        ref = np.array(brute_prefill(_lists(q), _lists(k), _lists(v), scale))
        assert np.max(np.abs(got - ref)) < 1e-12


def pin_mha_endpoint(o):
    """At Hkv = Hq the oracle is ordinary per-head attention: head h reads
    KV head h (study.greatitself.com, MHA endpoint)."""
    r = _rng(31)
    B, H, T, d = 2, 5, 7, 8
    q = r.standard_normal((B, H, d))
    k = r.standard_normal((B, H, T, d))
    v = r.standard_normal((B, H, T, d))
    got = o.decode(q, k, v, np.array([T, T]), 0.3)
    for b in range(B):
        for h in range(H):
            s = 0.3 * (k[b, h] @ q[b, h])
            w = np.exp(s - s.max())
            assert np.allclose(got[b, h], (w @ v[b, h]) / w.sum(), rtol=0, atol=1e-13)


def pin_mqa_endpoint(o):
    """At Hkv = 1 every query head reads the single KV head: permuting the
    query heads permutes the outputs the same way."""
    r = _rng(32)
    q = r.standard_normal((1, 6, 8))
    k = r.standard_normal((1, 1, 9, 8))
    v = r.standard_normal((1, 1, 9, 8))
    perm = np.array([3, 0, 5, 1, 4, 2])
    a = o.decode(q, k, v, np.array([9]), 0.5)
    b = o.decode(q[:, perm], k, v, np.array([9]), 0.5)
    assert np.array_equal(a[:, perm], b)


# -- exact special cases and invariants ---------------------------------------

def pin_special_cases(o):
    """K = 0 gives the mean of V; one token gives V[0] exactly; scale 0 gives
    the mean; an empty sequence gives zeros; scores far apart select the top
    value (needs the max subtraction: exp(1000) overflows otherwise)."""
    r = _rng(41)
    B, Hq, Hkv, T, d = 2, 4, 2, 6, 8
    q = r.standard_normal((B, Hq, d))
    k = r.standard_normal((B, Hkv, T, d))
    v = r.standard_normal((B, Hkv, T, d))
    lens = np.array([T, 3])
    mean = o.decode(q, np.zeros_like(k), v, lens, 0.7)
    zero_scale = o.decode(q, k, v, lens, 0.0)
    for b in range(B):
        for h in range(Hq):
            ref = v[b, h // 2, :lens[b]].mean(axis=0)
            assert np.allclose(mean[b, h], ref, rtol=0, atol=1e-14)
            assert np.allclose(zero_scale[b, h], ref, rtol=0, atol=1e-14)
    one = o.decode(q, k, v, np.array([1, 1]), 0.7)
    for h in range(Hq):
        assert np.array_equal(one[0, h], v[0, h // 2, 0]) and np.array_equal(one[1, h], v[1, h // 2, 0])
    empty, lse = o.decode(q, k, v, np.array([0, 2]), 0.7, return_lse=True)
    assert np.all(empty[0] == 0.0) and np.all(np.isneginf(lse[0])) and np.all(np.isfinite(lse[1]))
    # one-hot: key 4 aligned with q at a huge scale
    qq = np.zeros((1, 1, 4)); qq[0, 0, 0] = 1.0
    kk = np.zeros((1, 1, 6, 4)); kk[0, 0, :, 0] = [0.0, 0.1, -0.2, 0.3, 1.0, 0.5]
    vv = r.standard_normal((1, 1, 6, 4))
    top = o.decode(qq, kk, vv, np.array([6]), 2000.0)
    assert np.isfinite(top).all() and np.allclose(top[0, 0], vv[0, 0, 4], rtol=0, atol=1e-300)


def pin_causal_structure(o):
    """Prefill row 0 sees only key 0 (output V[0] exactly); the last row equals
    decode over all N tokens; changing keys/values after row i leaves rows
    0..i unchanged (lower-triangular mask, anrans.github.io)."""
    r = _rng(51)
    B, Hq, Hkv, N, d = 1, 4, 2, 7, 8
    q = r.standard_normal((B, Hq, N, d))
    k = r.standard_normal((B, Hkv, N, d))
    v = r.standard_normal((B, Hkv, N, d))
    out = o.prefill_causal(q, k, v, 0.35)
    for h in range(Hq):
        assert np.array_equal(out[0, h, 0], v[0, h // 2, 0])
    last = o.decode(q[:, :, N - 1], k, v, np.array([N]), 0.35)
    assert np.allclose(out[:, :, N - 1], last, rtol=0, atol=1e-14)
    i = 3
    k2, v2 = k.copy(), v.copy()
    k2[:, :, i + 1:] += 5.0
    v2[:, :, i + 1:] -= 3.0
    out2 = o.prefill_causal(q, k2, v2, 0.35)
    assert np.array_equal(out[:, :, :i + 1], out2[:, :, :i + 1])
    assert not np.allclose(out[:, :, i + 1:], out2[:, :, i + 1:])


def pin_prefill_rows_match(o):
    """Selected-row prefill equals the full computation."""
    r = _rng(52)
    q = r.standard_normal((1, 6, 10, 8))
    k = r.standard_normal((1, 2, 10, 8))
    v = r.standard_normal((1, 2, 10, 8))
    full, lse = o.prefill_causal(q, k, v, 0.4, return_lse=True)
    rows = [0, 4, 9]
    part, plse = o.prefill_causal_rows(q[0, 5, rows], k[0], v[0], rows, 5, 6, 0.4)
    assert np.allclose(part, full[0, 5, rows], rtol=0, atol=1e-14)
    assert np.allclose(plse, lse[0, 5, rows], rtol=0, atol=1e-14)


def pin_decode_one_matches(o):
    r = _rng(53)
    q = r.standard_normal((2, 8, 4))
    k = r.standard_normal((2, 2, 9, 4))
    v = r.standard_normal((2, 2, 9, 4))
    lens = np.array([9, 4])
    full, lse = o.decode(q, k, v, lens, 0.5, return_lse=True)
    for b in range(2):
        for h in range(8):
            one, l1 = o.decode_one(q[b, h], k[b], v[b], lens[b], h, 8, 0.5)
            assert np.allclose(one, full[b, h], rtol=0, atol=1e-14) and abs(l1 - lse[b, h]) < 1e-13


def pin_distinct_queries(o):
    """Distinct queries in one group give distinct outputs over shared K/V;
    identical queries give identical outputs (lihaoran.work)."""
    r = _rng(61)
    q = r.standard_normal((1, 4, 8))
    q[0, 1] = q[0, 0]
    k = r.standard_normal((1, 1, 12, 8))
    v = r.standard_normal((1, 1, 12, 8))
    out = o.decode(q, k, v, np.array([12]), 0.35)
    assert np.array_equal(out[0, 0], out[0, 1])
    assert not np.allclose(out[0, 0], out[0, 2])


def pin_convex_hull_and_permutation(o):
    """Each output coordinate lies within the range of the attended values;
    permuting the cached tokens (K and V together) leaves decode unchanged."""
    r = _rng(71)
    q = r.standard_normal((2, 4, 8)) * 3
    k = r.standard_normal((2, 2, 20, 8))
    v = r.standard_normal((2, 2, 20, 8))
    lens = np.array([20, 13])
    out = o.decode(q, k, v, lens, 0.35)
    for b in range(2):
        for h in range(4):
            vv = v[b, h // 2, :lens[b]]
            assert np.all(out[b, h] >= vv.min(axis=0) - 1e-12) and np.all(out[b, h] <= vv.max(axis=0) + 1e-12)
    perm = r.permutation(20)
    out2 = o.decode(q[:1], k[:1, :, perm], v[:1, :, perm], np.array([20]), 0.35)
    assert np.allclose(out2, out[:1], rtol=0, atol=1e-13)


def pin_distinct_kv_heads_matter(o):
    """With distinct K/V per KV head, swapping the two KV heads changes which
    query heads see which data (catches a wrong mapping that a test with
    identical heads would miss; study.greatitself.com)."""
    r = _rng(81)
    q = r.standard_normal((1, 4, 8))
    k = r.standard_normal((1, 2, 10, 8))
    v = r.standard_normal((1, 2, 10, 8))
    a = o.decode(q, k, v, np.array([10]), 0.35)
    b = o.decode(q[:, [2, 3, 0, 1]], k[:, ::-1], v[:, ::-1], np.array([10]), 0.35)
    assert np.array_equal(a[:, [2, 3, 0, 1]], b)
    # query head 1 must read KV head 0
    ref = o.decode(q[:, 1:2], k[:, 0:1], v[:, 0:1], np.array([10]), 0.35)
    assert np.allclose(a[:, 1:2], ref, rtol=0, atol=1e-15)


ATTENTION_PINS = [
    pin_mapping_examples, pin_mapping_endpoints, pin_rejects_irregular_grouping,
    pin_expand_is_consecutive,
    pin_two_queries_closed_form, pin_grouped_rows_equivalence, pin_brute_decode,
    pin_brute_prefill, pin_mha_endpoint, pin_mqa_endpoint, pin_special_cases,
    pin_causal_structure, pin_prefill_rows_match, pin_decode_one_matches,
    pin_distinct_queries, pin_convex_hull_and_permutation, pin_distinct_kv_heads_matter,
]
