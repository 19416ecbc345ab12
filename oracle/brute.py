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


def attention_row_biased(q, keys, values, tau, bias):
    """One query with an additive term per key on the scaled scores:
    s_j = q . k_j / tau + bias_j, a_j = e^{s_j} / sum_i e^{s_i} (no max
    shift), o = sum_j a_j v_j with values of any width.  Returns (o, lse)."""
    s = [math.fsum(qt * kt for qt, kt in zip(q, k)) / tau + b for k, b in zip(keys, bias)]
    e = [math.exp(x) for x in s]
    Z = math.fsum(e)
    width = len(values[0])
    o = [math.fsum(e[j] / Z * values[j][t] for j in range(len(values))) for t in range(width)]
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


def attention_grad(q, k, v, dout, causal=False, key_lens=None, tau=None):
    """Gradients (dq, dk, dv) of a loss L with dL/d(out) = ``dout``.

    Written out with the full Jacobian matrix of the weights, as the proof
    section (証明) of the formula page prints it: da_j/ds_l = a_j (delta_jl -
    a_l).  For every query row: dL/da_j = dout . v_j (from o = sum_j a_j v_j),
    dL/ds_l = sum_j dL/da_j * J[j][l], then dL/dq = sum_l dL/ds_l k_l / tau,
    dL/dk_l += dL/ds_l q / tau and dL/dv_j += a_j dout.  Nested lists in and
    out, shapes as in :func:`attention`.
    """
    B, H = len(q), len(q[0])
    d = len(q[0][0][0])
    if tau is None:
        tau = math.sqrt(d)
    dq = [[[[0.0] * d for _ in q[b][h]] for h in range(H)] for b in range(B)]
    dk = [[[[0.0] * d for _ in k[b][h]] for h in range(H)] for b in range(B)]
    dv = [[[[0.0] * d for _ in v[b][h]] for h in range(H)] for b in range(B)]
    for b in range(B):
        for h in range(H):
            Lk = len(k[b][h])
            # per key, the list of terms of dk and dv, summed at the end
            tk = [[[] for _ in range(d)] for _ in range(Lk)]
            tv = [[[] for _ in range(d)] for _ in range(Lk)]
            for i in range(len(q[b][h])):
                n = Lk
                if key_lens is not None:
                    n = min(n, max(0, int(key_lens[b])))
                if causal:
                    n = min(n, i + 1)
                if n == 0:
                    continue
                qi = [float(x) for x in q[b][h][i]]
                gi = [float(x) for x in dout[b][h][i]]
                s = [math.fsum(qi[t] * float(k[b][h][j][t]) for t in range(d)) / tau for j in range(n)]
                e = [math.exp(x) for x in s]
                Z = math.fsum(e)
                a = [x / Z for x in e]
                da = [math.fsum(gi[t] * float(v[b][h][j][t]) for t in range(d)) for j in range(n)]
                jac = [[a[j] * ((1.0 if j == l else 0.0) - a[l]) for l in range(n)] for j in range(n)]
                ds = [math.fsum(da[j] * jac[j][l] for j in range(n)) for l in range(n)]
                dq[b][h][i] = [math.fsum(ds[l] * float(k[b][h][l][t]) for l in range(n)) / tau
                               for t in range(d)]
                for l in range(n):
                    for t in range(d):
                        tk[l][t].append(ds[l] * qi[t] / tau)
                        tv[l][t].append(a[l] * gi[t])
            for j in range(Lk):
                dk[b][h][j] = [math.fsum(tk[j][t]) for t in range(d)]
                dv[b][h][j] = [math.fsum(tv[j][t]) for t in range(d)]
    return dq, dk, dv
