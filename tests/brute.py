"""Brute-force evaluation of the gated FFN with explicit index loops.

Independent of the oracle: every contraction is a Python loop over named
indices, so an operand transposed or an index swapped in the oracle shows
up as a mismatch. Tiny shapes only.
"""
from __future__ import annotations

import math


def _dot(row, vec):
    s = 0.0
    for a, b in zip(row, vec):
        s += a * b
    return s


def gate_row(wl, t):
    """g_i for token t: full gate, or U (V x) for the low-rank gate."""
    x = [float(v) for v in wl.x[t]]
    if wl.w_gate is not None:
        return [_dot(wl.w_gate[i], x) for i in range(wl.f)]
    inner = [_dot(wl.v[j], x) for j in range(wl.rank)]
    return [_dot(wl.u[i], inner) for i in range(wl.f)]


def act(z, kind):
    if kind == "relu":
        return z if z > 0.0 else 0.0
    return z / (1.0 + math.exp(-z))


def brute_forward(wl, k=None, bias=None, tau=None, dense=False):
    """y[t][o] for every token, plus the per-token active lists."""
    k = wl.k if k is None else k
    b = list(wl.bias_per_token() if bias is None else bias)
    taus = None
    if wl.sel == "thresh":
        taus = list(wl.tau if tau is None else tau)
    d_out = wl.w_down.shape[0]
    ys, actives = [], []
    for t in range(wl.m):
        x = [float(v) for v in wl.x[t]]
        g = gate_row(wl, t)
        z = [g[i] + b[t] for i in range(wl.f)]
        u = [_dot(wl.w_up[i], x) for i in range(wl.f)]
        if wl.sel == "topk":
            h = [act(z[i], wl.act) * u[i] for i in range(wl.f)]
            if dense:
                chosen = list(range(wl.f))
            else:
                c = [math.sqrt(sum(wl.w_down[o][i] ** 2 for o in range(d_out))) for i in range(wl.f)]
                s = [abs(h[i]) * c[i] for i in range(wl.f)]
                ranked = sorted(range(wl.f), key=lambda i: (-s[i], i))
                chosen = sorted(ranked[:k])
        else:
            cut = 0.0 if wl.sel == "bias" else max(taus[t], 0.0)
            chosen = [i for i in range(wl.f) if z[i] > cut]
            h = [z[i] * u[i] if z[i] > cut else 0.0 for i in range(wl.f)]
        y = [sum(wl.w_down[o][i] * h[i] for i in chosen) for o in range(d_out)]
        ys.append(y)
        actives.append(chosen)
    return ys, actives
