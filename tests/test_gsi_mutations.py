"""Planted mistakes in the GSI oracle must be caught by its pins (CPU only)."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import gsi_oracle as G
from tests import test_gsi_pins as P


def _pins_pass() -> bool:
    checks = [
        P.test_gsi_hand_example,
        P.test_gsi_exact_tie_is_slow,
        lambda: [P.test_gsi_matches_loops(s, o) for s, o in ((0, True), (1, False))],
        P.test_gsi_eps_zero_is_dense,
        P.test_gsi_full_basis_is_dense,
        P.test_gsi_pythagoras_orthonormal_basis,
        lambda: P.test_gsi_theorem4_bound(0),
    ]
    for chk in checks:
        try:
            chk()
        except (AssertionError, ValueError, IndexError):
            return False
    return True


def test_unmutated_gsi_oracle_passes():
    assert _pins_pass()


def _project_variant(kind):
    orig = G.project

    def project(vk, x):
        vk = np.asarray(vk, dtype=np.float64)
        x = np.atleast_2d(np.asarray(x, dtype=np.float64))
        g = x @ vk
        r = x + g @ vk.T if kind == "sign" else x - g @ vk.T
        nr = np.sqrt(np.sum(r * r, axis=1))
        nx = np.sqrt(np.sum(x * x, axis=1))
        ng = np.sqrt(np.sum(g * g, axis=1))
        den = ng if kind == "denominator" else nx
        rho = np.zeros(x.shape[0]) if kind != "zero_slow" else np.ones(x.shape[0])
        nz = den > 0
        rho[nz] = (nr[nz] / den[nz]) ** (2 if kind == "squared" else 1)
        return g, r, rho

    return orig, project


@pytest.mark.parametrize("kind", ["sign", "denominator", "squared", "zero_slow"])
def test_mutated_projection_is_caught(monkeypatch, kind):
    _, project = _project_variant(kind)
    monkeypatch.setattr(G, "project", project)
    assert not _pins_pass()


def test_non_strict_threshold_is_caught(monkeypatch):
    monkeypatch.setattr(G, "slow_tokens",
                        lambda rho, eps: np.nonzero(np.asarray(rho) > float(eps))[0].astype(np.int64))
    assert not _pins_pass()


def test_ungated_fast_path_is_caught(monkeypatch):
    """Dropping the gate (every token fast: static projection)."""
    monkeypatch.setattr(G, "slow_tokens", lambda rho, eps: np.zeros(0, dtype=np.int64))
    assert not _pins_pass()


def test_image_from_leading_columns_is_caught(monkeypatch):
    """The fast path reading W's first k columns instead of W V_k."""
    monkeypatch.setattr(G, "image", lambda w, vk: np.asarray(w, dtype=np.float64)[:, :np.asarray(vk).shape[1]])
    assert not _pins_pass()


def test_transposed_image_product_is_caught(monkeypatch):
    orig = G.forward

    def forward(w, img, vk, x, eps):
        g, _, rho = G.project(vk, x)
        slow = G.slow_tokens(rho, eps)
        img = np.asarray(img, dtype=np.float64)
        y = g @ img.T[::-1]                    # rows of the image in the wrong order
        if slow.size:
            y[slow] = G.dense(w, np.atleast_2d(np.asarray(x, dtype=np.float64))[slow])
        return y, rho, slow

    monkeypatch.setattr(G, "forward", forward)
    assert not _pins_pass()
    monkeypatch.setattr(G, "forward", orig)
