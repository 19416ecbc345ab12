"""Per-query brute force for tiny shapes (pure Python, no numpy arithmetic).

TEST INFRASTRUCTURE ONLY (see the ``oracle`` package docstring).

This is the second, even plainer route to the same numbers as the C oracle.
It applies the weights exactly as the proof section (証明) of the formula page
"トランスフォーマーの注意機構" prints them, with no shift by the maximum:

    s_j = (q . k_j) / tau                 (first display; tau = sqrt(d_k))
    a_j = e^{s_j} / sum_i e^{s_i}         (second display)
    o   = sum_j a_j v_j                   (third display)
    lse = log sum_i e^{s_i}               ("広がる学問 / 数学" paragraph)

Sums use ``math.fsum`` so the result is correctly rounded per sum.  Only for
shapes small enough that e^{s} cannot overflow.
"""
from __future__ import annotations

import math


def attention_row(q, keys, values, tau=None):
    """One query over a list of (key, value) pairs.  Returns (o, lse)."""
    d = len(q)
    if tau is None:
        tau = math.sqrt(d)
    if len(keys) == 0:
        return [0.0] * len(values[0] if values else q), -math.inf
    s = [math.fsum(qt * kt for qt, kt in zip(q, k)) / tau for k in keys]
    e = [math.exp(x) for x in s]
    Z = math.fsum(e)
    a = [x / Z for x in e]
    width = len(values[0])
    o = [math.fsum(a[j] * values[j][t] for j in range(len(values))) for t in range(width)]
    return o, math.log(Z)


def attention(q, k, v, causal=False, key_lens=None, tau=None):
    """Nested lists / arrays q[B][H][Lq][d], k and v [B][H][Lk][d].

    Returns (out[B][H][Lq][d], lse[B][H][Lq]) as nested lists of floats.
    Masks as in the C oracle: key j is dropped if j >= key_lens[b] or, when
    ``causal``, if j > i.
    """
    out, lse = [], []
    for b in range(len(q)):
        ob, lb = [], []
        for h in range(len(q[b])):
            oh, lh = [], []
            Lk = len(k[b][h])
            for i in range(len(q[b][h])):
                n = Lk
                if key_lens is not None:
                    n = min(n, max(0, int(key_lens[b])))
                if causal:
                    n = min(n, i + 1)
                qi = [float(x) for x in q[b][h][i]]
                keys = [[float(x) for x in k[b][h][j]] for j in range(n)]
                vals = [[float(x) for x in v[b][h][j]] for j in range(n)]
                if n == 0:
                    o, l = [0.0] * len(qi), -math.inf
                else:
                    o, l = attention_row(qi, keys, vals, tau)
                oh.append(o)
                lh.append(l)
            ob.append(oh)
            lb.append(lh)
        out.append(ob)
        lse.append(lb)
    return out, lse
