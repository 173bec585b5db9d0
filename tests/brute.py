"""Scalar brute force for tiny attention problems, in pure Python.

Test infrastructure: an independent restatement of the definition used to pin
the numpy oracle.  No arrays, no repeat, no vectorised softmax: every score is
a plain sum of products, the KV head is picked by index (query head h reads
KV head h // g), and sums use math.fsum.
"""
import math


def _attend(qvec, keys, values, scale):
    scores = [scale * math.fsum(a * b for a, b in zip(qvec, key)) for key in keys]
    top = max(scores)
    weights = [math.exp(s - top) for s in scores]
    total = math.fsum(weights)
    d = len(values[0])
    return [math.fsum(w * val[c] for w, val in zip(weights, values)) / total for c in range(d)]


def brute_decode(q, k, v, seq_lens, scale):
    """q[b][h][i]; k, v [b][kv][t][i]; returns out[b][h][i] as nested lists."""
    B, Hq = len(q), len(q[0])
    Hkv = len(k[0])
    g = Hq // Hkv
    out = []
    for b in range(B):
        T = int(seq_lens[b])
        rows = []
        for h in range(Hq):
            kv = h // g
            if T == 0:
                rows.append([0.0] * len(q[b][h]))
                continue
            keys = [list(k[b][kv][t]) for t in range(T)]
            vals = [list(v[b][kv][t]) for t in range(T)]
            rows.append(_attend(list(q[b][h]), keys, vals, scale))
        out.append(rows)
    return out


def brute_prefill(q, k, v, scale):
    """q[b][h][i][c]; k, v [b][kv][j][c]; causal (key j <= query i)."""
    B, Hq, N = len(q), len(q[0]), len(q[0][0])
    Hkv = len(k[0])
    g = Hq // Hkv
    out = []
    for b in range(B):
        heads = []
        for h in range(Hq):
            kv = h // g
            rows = []
            for i in range(N):
                keys = [list(k[b][kv][j]) for j in range(i + 1)]
                vals = [list(v[b][kv][j]) for j in range(i + 1)]
                rows.append(_attend(list(q[b][h][i]), keys, vals, scale))
            heads.append(rows)
        out.append(heads)
    return out


def brute_decode_paged(q, k_pages, v_pages, block_table, seq_lens, page_size, scale):
    """Decode through a block table: token t of sequence b is row t % page_size
    of page block_table[b][t // page_size]; pools are [page][kv][row][i]."""
    B, Hq = len(q), len(q[0])
    Hkv = len(k_pages[0])
    g = Hq // Hkv
    out = []
    for b in range(B):
        T = int(seq_lens[b])
        rows = []
        for h in range(Hq):
            kv = h // g
            keys, vals = [], []
            for t in range(T):
                page = int(block_table[b][t // page_size])
                keys.append(list(k_pages[page][kv][t % page_size]))
                vals.append(list(v_pages[page][kv][t % page_size]))
            rows.append(_attend(list(q[b][h]), keys, vals, scale) if T else [0.0] * len(q[b][h]))
        out.append(rows)
    return out


def e4m3_scalar(code):
    """One OCP E4M3 code as a Python float (math.ldexp on the bit fields)."""
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 7
    if e == 0xF and m == 7:
        return math.nan
    if e == 0:
        return sign * math.ldexp(m, -9)
    return sign * math.ldexp(8 + m, e - 10)
