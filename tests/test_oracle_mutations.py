"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case monkeypatches one oracle step with a plausible bug and runs the
pin checks; at least one must fail. This shows the pins constrain every
step, not just the happy path.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import ffn_oracle as O
from tests import test_oracle_pins as P


def _pins_pass() -> bool:
    checks = [
        lambda: [P.test_forward_matches_bruteforce(*c) for c in P.SMALL],
        lambda: P.test_wina_hand_example(),
        lambda: [P.test_wina_lemma31_optimal_for_orthogonal_columns(s) for s in (0, 1)],
        lambda: P.test_cut_is_strict_exact_tie_inactive(),
        lambda: [P.test_twell_roundtrip(*c) for c in P.SMALL],
        lambda: P.test_topk_tie_break_lower_index(),
        lambda: P.test_lowrank_bruteforce_distinct_factors(),
        lambda: P.test_input_wina_hand_example(),
        lambda: P.test_input_wina_lemma31_optimal_for_orthogonal_columns(),
        lambda: P.test_input_equal_norms_is_magnitude_topk(),
        lambda: P.test_input_keep_all_equals_full_gate(),
    ]
    for chk in checks:
        try:
            chk()
        except (AssertionError, ValueError, IndexError):
            return False
    return True


def test_unmutated_oracle_passes():
    assert _pins_pass()


_orig_gate = O.gate_preactivation
_orig_pack = O.twell_pack
_orig_topk = O.topk_lower_index


def _gate_rounds_intermediate(x, w_gate=None, u=None, v=None):
    if w_gate is not None:
        return _orig_gate(x, w_gate=w_gate)
    t = np.asarray(x) @ np.asarray(v).T
    t = t.astype(np.float32).astype(np.float64)
    return t @ np.asarray(u).T


def _gate_sign(x, w_gate=None, u=None, v=None):
    return -_orig_gate(x, w_gate, u, v)


def _gate_drops_column(x, w_gate=None, u=None, v=None):
    x = np.array(x, dtype=np.float64)
    x[:, -1] = 0.0
    return _orig_gate(x, w_gate, u, v)


def _mask_inclusive(z, cut):
    z = np.asarray(z, dtype=np.float64)
    cut = np.asarray(cut, dtype=np.float64)
    return z >= cut.reshape(-1, 1) if cut.ndim == 1 else z >= cut


def _norms_l1(w_down):
    return np.sum(np.abs(np.asarray(w_down, dtype=np.float64)), axis=0)


def _scores_h_only(h, col_norms):
    return np.abs(np.asarray(h, dtype=np.float64))


def _topk_higher_index(s_row, k):
    order = sorted(range(len(s_row)), key=lambda i: (-s_row[i], -i))
    return np.array(sorted(order[:k]), dtype=np.int64)


def _pack_off_by_one(mask, values, T, E, f32_values):
    cnt, idx, val = _orig_pack(mask, values, T, E, f32_values)
    live = idx != O.IDX_PAD
    idx = idx.copy()
    idx[live] = idx[live] + 1
    return cnt, idx, val


def _pack_values_truncated(mask, values, T, E, f32_values):
    v = np.asarray(values, dtype=np.float64)
    return _orig_pack(mask, np.trunc(v * 64) / 64, T, E, f32_values)


def _up_transposed_rows(x, w_up):
    return np.asarray(x, dtype=np.float64) @ np.asarray(w_up, dtype=np.float64)[::-1].T


def _down_without_h(h_active, cols, w_down):
    w = np.asarray(w_down, dtype=np.float64)
    return w[:, cols].sum(axis=1) if len(cols) else np.zeros(w.shape[0])


MUTATIONS = {
    "lowrank_intermediate_rounded": ("gate_preactivation", _gate_rounds_intermediate),
    "gate_sign_flipped": ("gate_preactivation", _gate_sign),
    "gate_drops_last_input": ("gate_preactivation", _gate_drops_column),
    "cut_inclusive": ("threshold_mask", _mask_inclusive),
    "wina_l1_norm": ("wina_column_norms", _norms_l1),
    "wina_hidden_only": ("wina_scores", _scores_h_only),
    "topk_ties_to_higher_index": ("topk_lower_index", _topk_higher_index),
    "pack_index_off_by_one": ("twell_pack", _pack_off_by_one),
    "pack_values_truncated": ("twell_pack", _pack_values_truncated),
    "up_rows_reversed": ("up_projection", _up_transposed_rows),
    "down_ignores_h": ("down_projection_sparse", _down_without_h),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    assert not _pins_pass(), f"planted mistake {name!r} passed every pin"


# ---------------------------------------------------------------------------
# input-side selection of the gate projection
# ---------------------------------------------------------------------------

_orig_in_norms = O.input_column_norms
_orig_in_scores = O.input_scores
_orig_in_gate = O.gate_preactivation_input_sparse


def _in_norms_of_rows(w):
    w = np.asarray(w, dtype=np.float64)
    r = np.sqrt(np.sum(w * w, axis=1))
    return np.resize(r, w.shape[1])


def _in_scores_magnitude_only(x, col_norms):
    return np.abs(np.asarray(x, dtype=np.float64)) + 0.0 * np.asarray(col_norms)


def _in_scores_squared_norm(x, col_norms):
    return np.abs(np.asarray(x, dtype=np.float64)) * np.asarray(col_norms, dtype=np.float64) ** 2


def _in_gate_ignores_selection(x, kept, w_gate=None, u=None, v=None):
    return O.gate_preactivation(x, w_gate, u, v)


def _in_gate_drops_last_kept(x, kept, w_gate=None, u=None, v=None):
    return _orig_in_gate(x, [k[:-1] if len(k) else k for k in kept], w_gate, u, v)


@pytest.mark.parametrize("name,attr,fn", [
    ("row norms for column norms", "input_column_norms", _in_norms_of_rows),
    ("|x| only", "input_scores", _in_scores_magnitude_only),
    ("squared column norm", "input_scores", _in_scores_squared_norm),
    ("selection ignored", "gate_preactivation_input_sparse", _in_gate_ignores_selection),
    ("last kept channel dropped", "gate_preactivation_input_sparse", _in_gate_drops_last_kept),
])
def test_input_mutation_caught(monkeypatch, name, attr, fn):
    monkeypatch.setattr(O, attr, fn)
    assert not _pins_pass(), f"planted mistake not caught: {name}"
