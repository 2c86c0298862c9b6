"""Brute-force twin of the oracle: scalar Python loops, ``math`` only.

TEST INFRASTRUCTURE ONLY.  It restates the same definition as
``oracle.materialized`` (see that module for the sources) one query row and one
key at a time, with no NumPy arithmetic, so that the two agree only if both
read the definition the same way.  Tiny shapes only.
"""

from __future__ import annotations

import math


def attend_row(q_row, keys, values, q_abs, valid, *, scale, causal, window,
               softcap, sink):
    """Output of one query row (list of floats) against lists of key/value rows."""
    logits = []
    kept = []
    for j in range(len(keys)):
        ok = 0 <= j < valid
        if causal and j > q_abs:
            ok = False
        if window != -1 and q_abs - j >= window:
            ok = False
        if not ok:
            continue
        x = scale * sum(a * b for a, b in zip(q_row, keys[j]))
        if softcap > 0:
            x = softcap * math.tanh(x / softcap)
        logits.append(x)
        kept.append(j)
    D = len(q_row)
    if not kept:
        return [0.0] * D
    top = max(logits)
    if sink is not None:
        top = max(top, sink)
    weights = [math.exp(x - top) for x in logits]
    denom = sum(weights)
    if sink is not None:
        denom += math.exp(sink - top)
    out = [0.0] * D
    for w, j in zip(weights, kept):
        for d in range(D):
            out[d] += w * values[j][d]
    return [o / denom for o in out]


def attention(q, k, v, q_offset, valid, *, scale, causal=True, window=-1,
              softcap=0.0, sink=None):
    """Same contract as ``oracle.materialized.attention`` (nested lists or arrays in,
    nested lists out: [B][Hq][Lq][D])."""
    B, Hq = len(q), len(q[0])
    Hkv = len(k[0])
    G = Hq // Hkv
    out = []
    for b in range(B):
        per_head = []
        for h in range(Hq):
            g = h // G
            keys = [list(map(float, row)) for row in k[b][g]]
            vals = [list(map(float, row)) for row in v[b][g]]
            s = None if sink is None else float(sink[h])
            rows = []
            for i, q_row in enumerate(q[b][h]):
                rows.append(attend_row(list(map(float, q_row)), keys, vals,
                                       int(q_offset[b]) + i, int(valid[b]),
                                       scale=scale, causal=causal, window=window,
                                       softcap=softcap, sink=s))
            per_head.append(rows)
        out.append(per_head)
    return out
