"""Pins of the GSI oracle (CPU only).

Each test checks the oracle against something other than itself: the hand
example printed in tests/golden/gsi_toy.txt, explicit index loops, the two
reductions to the dense product the method's definition fixes (eps = 0, and
a full basis k = d), Pythagoras for an orthonormal basis and the Theorem-4
bound of "Gated Subspace Inference for Transformer Acceleration", section 2.2.
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest

from oracle import gsi_oracle as G
from synth.gsi import make_gsi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "gsi_toy.txt")


def _parse_golden():
    w, toys, cur = [], {}, None
    for raw in open(GOLDEN, encoding="utf-8"):
        line = raw.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("["):
            cur = line.strip("[]")
            if cur != "w":
                toys[cur] = dict(tokens=[], eps=[])
            continue
        if cur == "w":
            w.append([float(v) for v in line.split()])
            continue
        toy = toys[cur]
        head, *rest = line.split()
        if head in ("basis", "image"):
            toy[head] = [float(v) for v in rest]
        elif head == "x":
            parts = [p.split() for p in line.split("|")]
            tok = {p[0]: [float(v) for v in p[1:]] for p in parts}
            toy["tokens"].append(tok)
        elif head == "eps":
            toy["eps"].append((float(rest[0]), [int(v) for v in rest[2:]]))
    return np.array(w), toys


# --------------------------------------------------------------- loops
def _loop_project(vk, x):
    d, k = len(vk), len(vk[0])
    g = [sum(vk[j][c] * x[j] for j in range(d)) for c in range(k)]
    r = [x[j] - sum(vk[j][c] * g[c] for c in range(k)) for j in range(d)]
    nr = math.sqrt(sum(v * v for v in r))
    nx = math.sqrt(sum(v * v for v in x))
    return g, r, (nr / nx if nx > 0 else 0.0)


def _loop_matvec(a, v):
    return [sum(a[o][j] * v[j] for j in range(len(v))) for o in range(len(a))]


def _loop_forward(w, vk, x, eps):
    k = len(vk[0])
    img = [[sum(w[o][j] * vk[j][c] for j in range(len(vk))) for c in range(k)] for o in range(len(w))]
    ys, rhos, slow = [], [], []
    for t, xt in enumerate(x):
        g, _, rho = _loop_project(vk, xt)
        rhos.append(rho)
        if rho < eps:
            ys.append(_loop_matvec(img, g))
        else:
            slow.append(t)
            ys.append(_loop_matvec(w, xt))
    return ys, rhos, slow


# --------------------------------------------------------------- pins
def test_gsi_hand_example():
    w, toys = _parse_golden()
    assert set(toys) == {"toy A", "toy B"}
    for toy in toys.values():
        vk = np.array(toy["basis"])[:, None]
        assert np.allclose(G.image(w, vk)[:, 0], toy["image"], rtol=0, atol=1e-12)
        x = np.array([t["x"] for t in toy["tokens"]])
        g, _, rho = G.project(vk, x)
        assert np.allclose(g[:, 0], [t["g"][0] for t in toy["tokens"]], rtol=0, atol=1e-12)
        assert np.allclose(rho, [t["rho"][0] for t in toy["tokens"]], rtol=0, atol=1e-12)
        assert np.allclose(G.dense(w, x), [t["dense"] for t in toy["tokens"]], rtol=0, atol=1e-12)
        img = np.array(toy["image"])[:, None]
        for eps, slow in toy["eps"]:
            y, _, sl = G.forward(w, img, vk, x, eps)
            assert sl.tolist() == slow, (eps, sl)
            for t, tok in enumerate(toy["tokens"]):
                want = tok["dense"] if t in slow else tok["fast"]
                assert np.allclose(y[t], want, rtol=0, atol=1e-12), (eps, t)


def test_gsi_exact_tie_is_slow():
    """rho == eps takes the full product (the fast path needs rho < eps)."""
    w, toys = _parse_golden()
    a = toys["toy A"]
    vk = np.array(a["basis"])[:, None]
    x = np.array([a["tokens"][0]["x"]])
    _, _, rho = G.project(vk, x)
    assert rho[0] == 0.8
    assert G.slow_tokens(rho, 0.8).tolist() == [0]
    assert G.slow_tokens(rho, np.nextafter(0.8, 1.0)).tolist() == []


@pytest.mark.parametrize("seed,ortho", [(0, True), (1, False), (2, True)])
def test_gsi_matches_loops(seed, ortho):
    rng = np.random.default_rng(seed)
    d, d_out, k, m = 7, 5, 3, 6
    w = rng.standard_normal((d_out, d))
    vk = np.linalg.qr(rng.standard_normal((d, k)))[0] if ortho else rng.standard_normal((d, k)) * 0.5
    x = rng.standard_normal((m, d))
    x[2] = 0.0
    eps = 0.6
    img = G.image(w, vk)
    y, rho, slow = G.forward(w, img, vk, x, eps)
    ys, rhos, sl = _loop_forward(w.tolist(), vk.tolist(), x.tolist(), eps)
    assert slow.tolist() == sl
    assert np.allclose(rho, rhos, rtol=1e-12, atol=1e-14)
    assert np.allclose(y, ys, rtol=1e-11, atol=1e-12)
    g, r, _ = G.project(vk, x)
    for t in range(m):
        gl, rl, _ = _loop_project(vk.tolist(), x[t].tolist())
        assert np.allclose(g[t], gl, atol=1e-12) and np.allclose(r[t], rl, atol=1e-12)


def test_gsi_eps_zero_is_dense():
    """eps = 0: no ratio is below it, every token takes y = W x."""
    wl = make_gsi(48, 20, 8, 9, eps=0.1, slow_frac=0.3, seed=3, zero_tokens=(4,))
    img = G.image(wl.w, wl.vk)
    y, _, slow = G.forward(wl.w, img, wl.vk, wl.x, 0.0)
    assert slow.tolist() == list(range(wl.m))
    want = [_loop_matvec(wl.w.tolist(), xt) for xt in wl.x.tolist()]
    assert np.allclose(y, want, rtol=1e-12, atol=1e-12)


def test_gsi_full_basis_is_dense():
    """k = d with V_k = I: r = 0, every token is fast and M g = W x."""
    rng = np.random.default_rng(5)
    d, d_out, m = 12, 7, 5
    w = rng.standard_normal((d_out, d))
    x = rng.standard_normal((m, d))
    vk = np.eye(d)
    img = G.image(w, vk)
    y, rho, slow = G.forward(w, img, vk, x, 1e-9)
    assert slow.size == 0 and np.all(rho == 0.0)
    want = [_loop_matvec(w.tolist(), xt) for xt in x.tolist()]
    assert np.allclose(y, want, rtol=1e-12, atol=1e-12)


def test_gsi_pythagoras_orthonormal_basis():
    rng = np.random.default_rng(6)
    d, k, m = 40, 6, 8
    q = np.linalg.qr(rng.standard_normal((d, k)))[0]
    x = rng.standard_normal((m, d))
    g, r, rho = G.project(q, x)
    assert np.allclose(np.sum(x * x, 1), np.sum(g * g, 1) + np.sum(r * r, 1), rtol=1e-12)
    assert np.allclose(r @ q, 0.0, atol=1e-12)           # residual orthogonal to the subspace
    assert np.allclose(rho ** 2, np.sum(r * r, 1) / np.sum(x * x, 1), rtol=1e-12)


@pytest.mark.parametrize("seed", [0, 1])
def test_gsi_theorem4_bound(seed):
    """Fast tokens: ||M g - W x|| = ||W r|| <= ||W||_2 ||r|| < ||W||_2 eps ||x||."""
    wl = make_gsi(64, 30, 8, 24, eps=0.3, slow_frac=0.3, seed=seed)
    img = G.image(wl.w, wl.vk)                            # exact image
    y, rho, slow = G.forward(wl.w, img, wl.vk, wl.x, wl.eps)
    norm_w = np.linalg.norm(wl.w, 2)                      # spectral norm (SVD)
    dense = G.dense(wl.w, wl.x)
    _, r, _ = G.project(wl.vk, wl.x)
    fast = [t for t in range(wl.m) if t not in set(slow.tolist())]
    assert fast and slow.size
    for t in fast:
        err = np.linalg.norm(y[t] - dense[t])
        assert abs(err - np.linalg.norm(wl.w @ r[t])) <= 1e-9 * max(err, 1.0)
        assert err <= norm_w * np.linalg.norm(r[t]) * (1 + 1e-12)
        assert err < norm_w * wl.eps * np.linalg.norm(wl.x[t])
    for t in slow.tolist():
        assert np.allclose(y[t], dense[t], rtol=1e-13, atol=1e-13)


def test_gsi_generator_ratios_near_targets():
    """The generator's tokens land near their target ratios, off the threshold."""
    wl = make_gsi(256, 16, 16, 40, eps=0.1, slow_frac=0.3, seed=2, zero_tokens=(7,))
    _, _, rho = G.project(wl.vk, wl.x)
    assert rho[7] == 0.0
    live = np.arange(wl.m) != 7
    assert np.all(np.abs(rho[live] - wl.target[live]) < 0.02)
    assert np.all((rho < wl.eps) == ~wl.slow_target)
