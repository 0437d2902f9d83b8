"""Pure-Python brute force attention for tiny shapes.

TEST INFRASTRUCTURE ONLY.  It pins the vectorised oracle in ``ref.py``: it is
written independently, element by element, with ``math.exp`` and
``math.fsum``, indexes the KV head as floor(h / G) directly instead of
repeating heads, and rotates each (i, i + D/2) pair on its own.  Nothing in
it is imported from ``ref.py``.
"""
from __future__ import annotations

import math


def _rot(vec, pos, theta):
    D = len(vec)
    half = D // 2
    out = list(vec)
    for i in range(half):
        ang = pos * theta ** (-2.0 * i / D)
        c, s = math.cos(ang), math.sin(ang)
        out[i] = vec[i] * c - vec[i + half] * s
        out[i + half] = vec[i + half] * c + vec[i] * s
    return out


def attend(qrow, keys, vals, scale):
    """softmax over the given keys of scale * <q, k>, applied to the values."""
    scores = [scale * math.fsum(a * b for a, b in zip(qrow, k)) for k in keys]
    m = max(scores)
    w = [math.exp(s - m) for s in scores]
    z = math.fsum(w)
    Dv = len(vals[0])
    return [math.fsum(w[j] * vals[j][d] for j in range(len(keys))) / z for d in range(Dv)]


def prefill(q, k, v, scale, causal, rope_theta=0.0):
    """q [B][Hq][S][D], k, v [B][Hkv][S][D] as nested lists -> nested list O."""
    B, Hq, S = len(q), len(q[0]), len(q[0][0])
    Hkv = len(k[0])
    G = Hq // Hkv
    out = []
    for b in range(B):
        ob = []
        for h in range(Hq):
            g = h // G
            oh = []
            for i in range(S):
                qi = q[b][h][i]
                if rope_theta > 0:
                    qi = _rot(qi, i, rope_theta)
                n = i + 1 if causal else S
                keys = []
                for j in range(n):
                    kj = k[b][g][j]
                    keys.append(_rot(kj, j, rope_theta) if rope_theta > 0 else kj)
                oh.append(attend(qi, keys, [v[b][g][j] for j in range(n)], scale))
            ob.append(oh)
        out.append(ob)
    return out


def decode(q, kc, vc, lengths, scale):
    """q [B][Hq][D], caches [B][Hkv][cap][D] -> O [B][Hq][D]."""
    B, Hq = len(q), len(q[0])
    G = Hq // len(kc[0])
    out = []
    for b in range(B):
        n = lengths[b]
        out.append([attend(q[b][h], kc[b][h // G][:n], vc[b][h // G][:n], scale)
                    if n > 0 else [0.0] * len(vc[b][0][0]) for h in range(Hq)])
    return out
