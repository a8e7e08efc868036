"""Pins of the oracle's backward pass (CPU only).

The gradients of L = sum_t <dy_t, y_t> with the forward pass's selection held
fixed are checked against (a) PyTorch autograd in fp64 on the dense masked
function (an independent evaluation), (b) central finite differences of the
oracle's own forward pass in random directions (exact for a function that is
linear in each weight with the mask fixed, up to rounding), and (c) explicit
index loops on a tiny case. Planted mistakes must fail them.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import ffn_oracle as O
from synth import draw_dy, make_workload

SMALL = [("c1", 4, {}), ("c2", 3, dict(d=128, f=512, T=128, E=64)),
         ("c5", 40, dict(d=128, f=1024, T=256, E=16))]   # the last one routes busy tokens


def _autograd(wl, dy, mask):
    import torch
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True)
    x, wg, wu, wd = t(wl.x), t(wl.w_gate), t(wl.w_up), t(wl.w_down)
    b = torch.tensor(wl.bias_per_token(), dtype=torch.float64).reshape(-1, 1)
    z = x @ wg.T + b
    a = z * torch.tensor(mask, dtype=torch.float64)
    y = (a * (x @ wu.T)) @ wd.T
    (y * torch.tensor(dy)).sum().backward()
    return {"dx": x.grad.numpy(), "dw_gate": wg.grad.numpy(), "dw_up": wu.grad.numpy(), "dw_down": wd.grad.numpy()}


def _rel(a, b):
    n = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (n if n > 0 else 1.0)


@pytest.mark.parametrize("cid,m,kw", SMALL)
def test_backward_matches_autograd(cid, m, kw):
    wl = make_workload(cid, m, 0, **kw)
    dy = draw_dy(wl, 1)
    fwd = O.forward(wl)
    g = O.backward(wl, dy, fwd)
    ref = _autograd(wl, dy, fwd["mask"])
    for k in ("dx", "dw_gate", "dw_up", "dw_down"):
        assert _rel(g[k], ref[k]) < 1e-12, k
    if cid == "c5":
        assert fwd["n_dense"] > 0                    # routed tokens take part with their full masks


@pytest.mark.parametrize("cid,m,kw", SMALL[:2])
def test_backward_finite_differences(cid, m, kw):
    wl = make_workload(cid, m, 0, **kw)
    dy = draw_dy(wl, 2)
    g = O.backward(wl, dy)
    rng = np.random.default_rng(7)

    def loss():
        return float(np.sum(dy * O.forward(wl)["y"]))

    for name, key in (("w_gate", "dw_gate"), ("w_up", "dw_up"), ("w_down", "dw_down"), ("x", "dx")):
        base = getattr(wl, name).copy()
        D = rng.standard_normal(base.shape)
        # small enough that no pre-activation crosses its cut (band delta);
        # L is quadratic in each argument with the mask fixed, so the central
        # difference is exact up to rounding
        h = 1e-6
        setattr(wl, name, base + h * D)
        lp = loss()
        setattr(wl, name, base - h * D)
        lm = loss()
        setattr(wl, name, base)
        fd = (lp - lm) / (2 * h)
        an = float(np.sum(g[key] * D))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_backward_loops_tiny():
    wl = make_workload("c1", 2, 3, d=8, f=16, T=16, E=16)
    dy = draw_dy(wl, 3)
    g = O.backward(wl, dy)
    d, f, m = wl.d, wl.f, wl.m
    b = wl.bias_per_token()
    for t in range(m):
        z = [sum(wl.w_gate[i][j] * wl.x[t][j] for j in range(d)) + b[t] for i in range(f)]
        u = [sum(wl.w_up[i][j] * wl.x[t][j] for j in range(d)) for i in range(f)]
        act = [z[i] > 0 for i in range(f)]
        dh = [sum(wl.w_down[o][i] * dy[t][o] for o in range(d)) for i in range(f)]
        for i in range(f):
            du = dh[i] * z[i] if act[i] else 0.0
            dz = dh[i] * u[i] if act[i] else 0.0
            assert abs(g["du"][t, i] - du) < 1e-12 and abs(g["dz"][t, i] - dz) < 1e-12
        for j in range(d):
            want = sum((dh[i] * z[i] * wl.w_up[i][j] + dh[i] * u[i] * wl.w_gate[i][j]) for i in range(f) if act[i])
            assert abs(g["dx"][t, j] - want) < 1e-11
    for i in range(f):
        for j in range(d):
            assert abs(g["dw_up"][i, j] - sum(g["du"][t, i] * wl.x[t][j] for t in range(m))) < 1e-11
            assert abs(g["dw_down"][j, i] - sum(dy[t][j] * g["h"][t, i] for t in range(m))) < 1e-11


def _pins_pass() -> bool:
    try:
        test_backward_matches_autograd(*SMALL[0])
        test_backward_loops_tiny()
    except AssertionError:
        return False
    return True


def _variant(kind):
    orig = O.backward

    def bwd(wl, dy, fwd=None):
        out = orig(wl, dy, fwd)
        x = np.asarray(wl.x, dtype=np.float64)
        fwd = O.forward(wl) if fwd is None else fwd
        a = np.where(fwd["mask"], fwd["z"], 0.0)
        u = O.up_projection(x, wl.w_up)
        dh = np.asarray(dy) @ np.asarray(wl.w_down)
        if kind == "dz_unmasked":
            dz = dh * u
            out["dz"] = dz
            out["dw_gate"] = dz.T @ x
            out["dx"] = out["du"] @ wl.w_up + dz @ wl.w_gate
        elif kind == "du_uses_u":
            du = dh * u * fwd["mask"]
            out["du"] = du
            out["dw_up"] = du.T @ x
            out["dx"] = du @ wl.w_up + out["dz"] @ wl.w_gate
        elif kind == "dx_no_gate_term":
            out["dx"] = out["du"] @ wl.w_up
        elif kind == "dw_down_transposed_h":
            out["dw_down"] = np.asarray(dy).T @ (a * 0 + out["h"][:, ::-1])
        return out

    return bwd


@pytest.mark.parametrize("kind", ["dz_unmasked", "du_uses_u", "dx_no_gate_term", "dw_down_transposed_h"])
def test_backward_mutations_caught(monkeypatch, kind):
    assert _pins_pass()
    monkeypatch.setattr(O, "backward", _variant(kind))
    assert not _pins_pass()


@pytest.mark.parametrize("cid,m,kw", SMALL)
def test_backward_sampled_matches_autograd_and_full(cid, m, kw):
    """The sampled evaluation used at full size equals autograd's rows (an
    independent evaluation) and the full oracle's rows."""
    wl = make_workload(cid, m, 0, **kw)
    dy = draw_dy(wl, 3)
    fwd = O.forward(wl)
    ref = _autograd(wl, dy, fwd["mask"])
    full = O.backward(wl, dy, fwd)
    rng = np.random.default_rng(11)
    tokens = np.sort(rng.choice(m, min(m, 3), replace=False))
    neurons = np.sort(rng.choice(wl.f, 9, replace=False))
    sm = O.backward_sampled(wl, dy, tokens, neurons)
    assert _rel(sm["dx"], ref["dx"][tokens]) < 1e-12
    assert _rel(sm["dw_gate"], ref["dw_gate"][neurons]) < 1e-12
    assert _rel(sm["dw_up"], ref["dw_up"][neurons]) < 1e-12
    assert _rel(sm["dw_down_nm"], ref["dw_down"][:, neurons].T) < 1e-12
    assert _rel(sm["dx"], full["dx"][tokens]) < 1e-12
    assert _rel(sm["dw_down_nm"], full["dw_down"][:, neurons].T) < 1e-12
