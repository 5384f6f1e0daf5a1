"""Pure-Python scalar oracle for hand-sized inputs.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Written independently
of ``oracle.c``: a token is found one at a time through ``resolve`` (the
logical position -> (physical block, offset) translation of "vLLM Internals:
PagedAttention, Continuous Batching, and Where the 2-4x Comes From", section
"PagedAttention: page tables, for KV"), and the softmax is taken straight
from the per-token equation of "Efficient Memory Management for Large
Language Model Serving with PagedAttention", §3.4 "PagedAttention Algorithm":
exponentials of the scaled scores, each divided by their sum (no max
subtraction, ``math.fsum`` for the sums).  Only for small scores and short
sequences: it is slow and can overflow on large scores by design.
"""
from __future__ import annotations

import math


def resolve(table_row, pos, block_size):
    """Logical token position -> (physical block id, offset in the block)."""
    logical, offset = divmod(pos, block_size)
    return int(table_row[logical]), offset


def _f(x):
    return float(x)


def attend_one(qv, keys, values, scale):
    """o = sum_j a_j v_j with a_j = exp(s_j) / sum_t exp(s_t), s_j = scale q.k_j."""
    n = len(keys)
    D = len(qv)
    if n == 0:
        return [0.0] * D, []
    e = [math.exp(scale * math.fsum(_f(qv[d]) * _f(k[d]) for d in range(D))) for k in keys]
    Z = math.fsum(e)
    a = [x / Z for x in e]
    o = [math.fsum(a[j] * _f(values[j][d]) for j in range(n)) for d in range(D)]
    return o, a


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, widen=float):
    """q [S][Hq][D], caches [NB][B][Hkv][D] (any nested indexables of values
    that ``widen`` turns into Python floats exactly).  Returns (out, weights)."""
    S = len(q)
    Hq = len(q[0])
    B = len(k_cache[0])
    Hkv = len(k_cache[0][0])
    G = Hq // Hkv
    out, weights = [], []
    for s in range(S):
        n = int(context_lens[s])
        row_o, row_a = [], []
        for h in range(Hq):
            g = h // G
            keys, vals = [], []
            for t in range(n):
                b, off = resolve(block_tables[s], t, B)
                keys.append([widen(x) for x in k_cache[b][off][g]])
                vals.append([widen(x) for x in v_cache[b][off][g]])
            o, a = attend_one([widen(x) for x in q[s][h]], keys, vals, scale)
            row_o.append(o)
            row_a.append(a)
        out.append(row_o)
        weights.append(row_a)
    return out, weights


def prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, widen=float):
    """Multi-token queries, one scalar at a time: q [rows][Hq][D]; sequence s
    owns rows query_start[s] .. query_start[s+1]-1, the last T of its n
    cached tokens; the chunk's r-th row sits at position n - T + r and
    attends to positions 0 .. n - T + r.  Returns out [rows][Hq][D]."""
    Hq = len(q[0])
    B = len(k_cache[0])
    Hkv = len(k_cache[0][0])
    G = Hq // Hkv
    out = [None] * len(q)
    for s in range(len(context_lens)):
        n = int(context_lens[s])
        lo, hi = int(query_start[s]), int(query_start[s + 1])
        for i in range(lo, hi):
            visible = n - (hi - lo) + (i - lo) + 1
            row = []
            for h in range(Hq):
                g = h // G
                keys, vals = [], []
                for t in range(visible):
                    b, off = resolve(block_tables[s], t, B)
                    keys.append([widen(x) for x in k_cache[b][off][g]])
                    vals.append([widen(x) for x in v_cache[b][off][g]])
                o, _ = attend_one([widen(x) for x in q[i][h]], keys, vals, scale)
                row.append(o)
            out[i] = row
    return out
