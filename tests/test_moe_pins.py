"""Pins of the mixture-of-experts combination in the oracle (CPU only).

Each expert is the pinned single-FFN oracle; what is new is the routing and
the weighted sum (LoPA page, "Model Casting and Quality at 90% Sparsity").
Checked against: a one-expert layer (equal to the plain FFN), explicit loops
over tokens and slots with the brute-force FFN, and relabelling the experts.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import ffn_oracle as O
from synth.moe import make_moe
from tests.brute import brute_forward

SMALL = dict(d=256, f=1024, rank=32, T=64, E=64)


def _loop_moe(mw):
    ys = [brute_forward(wl)[0] if wl.m else [] for wl in mw.experts]
    y = np.zeros((mw.m, mw.d))
    for t in range(mw.m):
        for s in range(mw.topk):
            e = int(mw.expert_ids[t, s])
            i = int(np.nonzero(mw.rows[e] == t)[0][0])
            assert int(mw.slots[e][i]) == s
            y[t] += mw.weights[t, s] * np.asarray(ys[e][i])
    return y


def test_moe_one_expert_is_the_ffn():
    mw = make_moe(5, n_experts=1, topk=1, seed=3, **SMALL)
    assert np.all(mw.weights == 1.0)
    y = O.moe_forward(mw)["y"]
    assert np.array_equal(y, O.forward(mw.experts[0])["y"])


@pytest.mark.parametrize("m,ne,k,seed", [(6, 4, 2, 0), (9, 3, 3, 1), (4, 5, 1, 2)])
def test_moe_matches_loops(m, ne, k, seed):
    mw = make_moe(m, n_experts=ne, topk=k, seed=seed, **SMALL)
    assert np.allclose(mw.weights.sum(axis=1), 1.0, atol=1e-6)
    for t in range(m):
        assert len(set(mw.expert_ids[t].tolist())) == k
    y = O.moe_forward(mw)["y"]
    assert np.allclose(y, _loop_moe(mw), rtol=1e-10, atol=1e-11)


def test_moe_relabelling_experts_keeps_y():
    mw = make_moe(7, n_experts=4, topk=2, seed=4, **SMALL)
    y = O.moe_forward(mw)["y"]
    perm = [2, 0, 3, 1]                        # new expert p holds old expert perm[p]
    inv = np.argsort(perm)
    mw.experts = [mw.experts[p] for p in perm]
    mw.rows = [mw.rows[p] for p in perm]
    mw.slots = [mw.slots[p] for p in perm]
    mw.expert_ids = inv[mw.expert_ids]
    assert np.allclose(O.moe_forward(mw)["y"], y, rtol=1e-13, atol=1e-14)


def test_moe_every_slot_counted_once():
    mw = make_moe(8, n_experts=4, topk=2, seed=5, **SMALL)
    total = sum(int(r.size) for r in mw.rows)
    assert total == mw.m * mw.topk
    pairs = {(int(t), int(s)) for r, sl in zip(mw.rows, mw.slots) for t, s in zip(r, sl)}
    assert pairs == {(t, s) for t in range(mw.m) for s in range(mw.topk)}


def _pins_pass() -> bool:
    try:
        test_moe_one_expert_is_the_ffn()
        test_moe_matches_loops(6, 4, 2, 0)
    except AssertionError:
        return False
    return True


def _combine_variant(kind):
    def combine(expert_y, rows, slots, weights, m, d):
        y = np.zeros((m, d))
        w = np.asarray(weights, dtype=np.float64)
        for e, (ye, r_e, s_e) in enumerate(zip(expert_y, rows, slots)):
            if kind == "first_expert_only" and e > 0:
                continue
            for i, (t, s) in enumerate(zip(r_e, s_e)):
                ww = 1.0 if kind == "unweighted" else w[int(t), 0 if kind == "slot0_weight" else int(s)]
                y[int(t)] += ww * np.asarray(ye[i], dtype=np.float64)
        return y
    return combine


@pytest.mark.parametrize("kind", ["unweighted", "slot0_weight", "first_expert_only"])
def test_moe_mutations_caught(monkeypatch, kind):
    assert _pins_pass()
    monkeypatch.setattr(O, "moe_combine", _combine_variant(kind))
    assert not _pins_pass()
