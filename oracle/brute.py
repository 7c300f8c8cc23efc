"""Pure-Python scalar twin of the oracle for tiny shapes.

TEST INFRASTRUCTURE ONLY.  Written with explicit loops and the ``math``
module so that it shares no vectorised code path with :mod:`oracle.dkv_oracle`;
the pins compare the two on tiny inputs.
"""
from __future__ import annotations

import math


def rope_neox_py(x, pos, theta):
    """Rotate-half RoPE of one vector (list of floats) at integer position pos."""
    D = len(x)
    half = D // 2
    y = [0.0] * D
    for i in range(half):
        f = theta ** (-(2.0 * i) / D)
        a = pos * f
        c, s = math.cos(a), math.sin(a)
        y[i] = x[i] * c - x[i + half] * s
        y[i + half] = x[i + half] * c + x[i] * s
    return y


def dot_py(a, b):
    acc = 0.0
    for x, y in zip(a, b):
        acc += x * y
    return acc


def matvec_rows_py(x, w):
    """x [hidden] times W [hidden][N] -> [N]."""
    n = len(w[0])
    out = [0.0] * n
    for i, xi in enumerate(x):
        row = w[i]
        for j in range(n):
            out[j] += xi * row[j]
    return out


def attention_py(q_rot, k, v, scale):
    """q_rot [Hq][D], k, v [N][Hkv][D] nested lists -> (o [Hq][D], lse [Hq])."""
    Hq = len(q_rot)
    Hkv = len(k[0])
    g = Hq // Hkv
    D = len(q_rot[0])
    outs, lses = [], []
    for h in range(Hq):
        kvh = h // g
        s = [scale * dot_py(q_rot[h], k[t][kvh]) for t in range(len(k))]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        z = sum(e)
        o = [0.0] * D
        for t in range(len(k)):
            w = e[t] / z
            for d in range(D):
                o[d] += w * v[t][kvh][d]
        outs.append(o)
        lses.append(m + math.log(z))
    return outs, lses


def merge_py(parts):
    """parts: list of (o [Hq][D], lse [Hq]) -> merged (o, lse)."""
    Hq = len(parts[0][1])
    D = len(parts[0][0][0])
    o = [[0.0] * D for _ in range(Hq)]
    lse = [-math.inf] * Hq
    for h in range(Hq):
        ls = [p[1][h] for p in parts]
        if all(x == -math.inf for x in ls):
            continue
        M = max(ls)
        ws = [0.0 if x == -math.inf else math.exp(x - M) for x in ls]
        tot = sum(ws)
        for (po, _), w in zip(parts, ws):
            for d in range(D):
                o[h][d] += w * po[h][d] / tot
        lse[h] = M + math.log(tot)
    return o, lse


def prefill_py(q_rot, k, v, pos, scale):
    """Causal prefill: q_rot [n][Hq][D] already rotated, row j at position pos[j]
    attends to tokens 0..pos[j] of k, v [N][Hkv][D]."""
    n = len(q_rot)
    outs, lses = [], []
    for j in range(n):
        o, l = attention_py(q_rot[j], k[:pos[j] + 1], v[:pos[j] + 1], scale)
        outs.append(o)
        lses.append(l)
    return outs, lses


def linear_py(x, w):
    """x [M][K] times W^T for W [N][K] (nested lists) -> [M][N]."""
    return [[dot_py(xm, wn) for wn in w] for xm in x]
