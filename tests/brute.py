"""Brute force at 50 significant digits (mpmath), for tiny inputs.

Written from the mathematical definitions, not from the oracle: softmax is
exp(s) / sum exp(s) with no max subtracted (at 50 digits nothing overflows),
sums run over the keys the join predicate admits (j <= i for the causal one),
and gradients are central finite differences of the loss sum(o^2)/2 with a
step far below float64 resolution.
"""
from __future__ import annotations

import mpmath
import numpy as np

mpmath.mp.dps = 50


def _mp(a):
    return [[mpmath.mpf(float(x)) for x in row] for row in np.asarray(a, dtype=np.float64)]


def causal(i, n):
    """Keys of query i under q.t >= k.t."""
    return list(range(i + 1))


def pairs(mask="causal", window=0, seg=None):
    """The list of keys query i may see, per join predicate: causal (j <= i),
    full (every key), window (j <= i and i - j < window); with segment ids,
    only the keys whose id equals the query's."""
    if mask == "causal":
        base = causal
    elif mask == "full":
        base = lambda i, n: list(range(n))
    elif mask == "window":
        base = lambda i, n: list(range(max(0, i - window + 1), i + 1))
    else:
        raise ValueError(mask)
    if seg is None:
        return base
    return lambda i, n: [j for j in base(i, n) if seg[j] == seg[i]]


def attention(q, k, v, scale=0.125, keys=causal):
    """(o, lse) of softmax attention for one head, as mpf nested lists; keys(i, n)
    lists the keys query i sees."""
    Q, K, V = _mp(q), _mp(k), _mp(v)
    return _attention_mp(Q, K, V, mpmath.mpf(scale), keys)


def _attention_mp(Q, K, V, scale, keys=causal):
    n, d = len(Q), len(Q[0])
    o, lse = [], []
    for i in range(n):
        js = keys(i, n)
        e = [mpmath.exp(mpmath.fsum(Q[i][t] * K[j][t] for t in range(d)) * scale) for j in js]
        z = mpmath.fsum(e)
        o.append([mpmath.fsum(e[a] / z * V[j][t] for a, j in enumerate(js))
                  for t in range(len(V[0]))])
        lse.append(mpmath.log(z))
    return o, lse


def to_np(x):
    return np.array([[float(a) for a in row] for row in x]) if isinstance(x[0], list) \
        else np.array([float(a) for a in x])


def loss_mp(Q, K, V, scale, keys=causal):
    o, _ = _attention_mp(Q, K, V, scale, keys)
    return mpmath.fsum(x * x for row in o for x in row) / 2


def grad_fd(q, k, v, scale=0.125, h="1e-20", keys=causal):
    """Central finite differences of loss = sum(o^2)/2 w.r.t. every q, k, v entry."""
    h = mpmath.mpf(h)
    scale = mpmath.mpf(scale)
    base = [_mp(q), _mp(k), _mp(v)]
    grads = []
    for which in range(3):
        a = base[which]
        g = np.zeros((len(a), len(a[0])))
        for r in range(len(a)):
            for c in range(len(a[0])):
                x0 = a[r][c]
                a[r][c] = x0 + h
                lp = loss_mp(*base, scale, keys)
                a[r][c] = x0 - h
                lm = loss_mp(*base, scale, keys)
                a[r][c] = x0
                g[r, c] = float((lp - lm) / (2 * h))
        grads.append(g)
    return tuple(grads)


def nw(tx, ty, sx, sy, sv, denom=0.25):
    """sum(w v) / sum(w), w = exp(-((tx-sx)^2 + (ty-sy)^2) / denom), no shift."""
    out = []
    S = [(mpmath.mpf(float(a)), mpmath.mpf(float(b)), mpmath.mpf(float(c)))
         for a, b, c in zip(sx, sy, sv)]
    dn = mpmath.mpf(denom)
    for x, y in zip(tx, ty):
        x, y = mpmath.mpf(float(x)), mpmath.mpf(float(y))
        w = [mpmath.exp(-((x - a) ** 2 + (y - b) ** 2) / dn) for a, b, _ in S]
        out.append(float(mpmath.fsum(wi * c for wi, (_, _, c) in zip(w, S)) / mpmath.fsum(w)))
    return np.array(out)
