"""Pure-Python scalar attention for tiny shapes.

TEST INFRASTRUCTURE ONLY.  A second, deliberately different route to the same
definition as ``oracle.attention`` (nested loops, ``math.exp`` and ``math.fsum``
on Python floats, its own walk over the block table) so that a slip in the
vectorised oracle shows up as a disagreement.  Inputs are plain nested lists
of floats and ints.
"""
from __future__ import annotations

import math


def _row(cache, block_row, j, block_size):
    phys = block_row[j // block_size]
    if phys < 0:
        raise IndexError("unallocated block")
    return cache[phys * block_size + (j % block_size)]


def decode(q, k_cache, v_cache, block_tables, context_lens, block_size, scale):
    """q[b][h][i], cache[slot][g][i] -> out[b][h][i] (Python floats)."""
    out = []
    for b, qb in enumerate(q):
        n = context_lens[b]
        hq = len(qb)
        hkv = len(k_cache[0])
        per = hq // hkv
        rows = []
        for h in range(hq):
            g = h // per
            if n == 0:
                rows.append([0.0] * len(qb[h]))
                continue
            keys = [_row(k_cache, block_tables[b], j, block_size)[g] for j in range(n)]
            vals = [_row(v_cache, block_tables[b], j, block_size)[g] for j in range(n)]
            rows.append(_attend(qb[h], keys, vals, scale))
        out.append(rows)
    return out


def prefill(q, k_cache, v_cache, cu_q, cu_k, block_tables, block_size, scale, causal):
    """q[row][h][i] packed by cu_q -> out[row][h][i]."""
    out = [None] * len(q)
    hkv = len(k_cache[0])
    for s in range(len(cu_q) - 1):
        lq = cu_q[s + 1] - cu_q[s]
        lk = cu_k[s + 1] - cu_k[s]
        for r in range(lq):
            qrow = q[cu_q[s] + r]
            hq = len(qrow)
            per = hq // hkv
            last = (lk - lq + r) if causal else (lk - 1)  # last visible key position
            rows = []
            for h in range(hq):
                g = h // per
                keys = [_row(k_cache, block_tables[s], j, block_size)[g] for j in range(last + 1)]
                vals = [_row(v_cache, block_tables[s], j, block_size)[g] for j in range(last + 1)]
                rows.append(_attend(qrow[h], keys, vals, scale) if keys else [0.0] * len(qrow[h]))
            out[cu_q[s] + r] = rows
    return out


def _attend(qv, keys, vals, scale):
    scores = [scale * math.fsum(a * b for a, b in zip(qv, kv)) for kv in keys]
    top = max(scores)
    ex = [math.exp(x - top) for x in scores]
    tot = math.fsum(ex)
    d = len(vals[0])
    return [math.fsum(ex[j] * vals[j][i] for j in range(len(vals))) / tot for i in range(d)]
