"""Pins of the CPU oracle to facts fixed outside it (CPU only).

Each test ties an oracle function to brute force, a closed form, an
invariant, a hand-computed example or an enumeration, so that a dropped
term, a wrong sign or index, or a transposed operand fails at least one.
"""
from __future__ import annotations

import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import ffn_oracle as O
from synth import Workload, make_workload, round_bf16, bf16_bits
from tests.brute import brute_forward

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small(cid, m, seed=0, **kw):
    return make_workload(cid, m, seed, **kw)


# reduced-size instances of every workload: several tiles, ragged token counts
SMALL = [
    ("c1", 3, dict(d=16, f=64, T=16, E=16)),
    ("c1", 3, dict(d=16, f=64, T=16, E=2)),
    ("c2", 5, dict(d=16, f=64, T=16, E=4)),
    ("c3", 3, dict(d=16, f=64, rank=4, T=16, E=4)),
    ("c4", 3, dict(d=16, f=64, T=16, E=16)),
    ("c5", 7, dict(d=16, f=64, T=32, E=6)),
]


# ---------------------------------------------------------------------------
# bf16 rounding: exact rational definition on the two neighbouring values
# ---------------------------------------------------------------------------

def _bf16_nearest_bruteforce(v: float) -> int:
    """bf16 bits of v by comparing exact distances to both neighbours."""
    if v == 0.0:
        return 0x8000 if math.copysign(1.0, v) < 0 else 0
    sign = 0x8000 if v < 0 else 0
    a = Fraction(abs(v))
    e = math.floor(math.log2(abs(v)))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - 7)
    lo = (a // ulp) * ulp
    hi = lo + ulp
    if a - lo < hi - a:
        r = lo
    elif a - lo > hi - a:
        r = hi
    else:
        r = lo if (lo / ulp) % 2 == 0 else hi
    f32 = np.float32(float(r)).view(np.uint32)
    return sign | int(f32 >> 16)


def test_bf16_rounding_matches_exact_definition():
    rng = np.random.default_rng(7)
    vals = list(rng.standard_normal(400) * 10.0 ** rng.integers(-3, 3, 400))
    # exact ties and near-ties at several binades
    for e in (-5, 0, 3):
        base = 2.0 ** e
        ulp = base * 2.0 ** -7
        for j in range(4):
            vals += [base + (j + 0.5) * ulp, -(base + (j + 0.5) * ulp),
                     base + (j + 0.5) * ulp + 2.0 ** (e - 40), base + (j + 0.5) * ulp - 2.0 ** (e - 40)]
    vals = np.array(vals, dtype=np.float64)
    want = np.array([_bf16_nearest_bruteforce(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(O.bf16_rne_bits(vals), want)
    # the generator's independent rounding agrees with the definition too
    assert np.array_equal(bf16_bits(round_bf16(vals)), want)


# ---------------------------------------------------------------------------
# brute force: whole forward pass on tiny shapes, every mode
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cid,m,kw", SMALL)
def test_forward_matches_bruteforce(cid, m, kw):
    wl = small(cid, m, **kw)
    ref = O.forward(wl)
    ys, actives = brute_forward(wl)
    y = np.array(ys)
    assert np.allclose(ref["y"], y, rtol=1e-12, atol=1e-12 * max(1.0, np.abs(y).max()))
    for t in range(m):
        assert list(np.nonzero(ref["mask"][t])[0]) == actives[t]


@pytest.mark.parametrize("cid,m,kw", SMALL)
def test_dense_forward_matches_bruteforce(cid, m, kw):
    wl = small(cid, m, **kw)
    ys, _ = brute_forward(wl, dense=True)
    assert np.allclose(O.dense_forward(wl), np.array(ys), rtol=1e-12, atol=1e-12)


def test_lowrank_bruteforce_distinct_factors():
    # U (V x) with r < d: a transposed factor or a skipped stage changes g
    wl = small("c3", 2, d=12, f=32, rank=3, T=16, E=16)
    g = O.gate_preactivation(wl.x, u=wl.u, v=wl.v)
    from tests.brute import gate_row
    for t in range(2):
        assert np.allclose(g[t], gate_row(wl, t), rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# invariants and special cases
# ---------------------------------------------------------------------------

def test_sparsity_zero_equals_dense_relu_ffn():
    wl = small("c2", 3, d=16, f=64, T=16, E=16)
    big = np.full(3, 1.0e6)                      # every z > 0: a = z everywhere
    ref = O.forward(wl, bias=big)
    assert ref["mask"].all()
    x, wu, wd = wl.x, wl.w_up, wl.w_down
    z = x @ wl.w_gate.T + 1.0e6
    dense = (z * (x @ wu.T)) @ wd.T
    assert np.allclose(ref["y"], dense, rtol=1e-12)


def test_topk_all_equals_dense_silu_ffn():
    wl = small("c4", 2, d=16, f=64, T=16, E=16)
    ref = O.forward(wl, k=wl.f)
    z = wl.x @ wl.w_gate.T
    dense = ((z / (1 + np.exp(-z))) * (wl.x @ wl.w_up.T)) @ wl.w_down.T
    assert np.allclose(ref["y"], dense, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("how", ["bias", "topk0", "zero_x"])
def test_all_masked_gives_exact_zero(how):
    if how == "topk0":
        wl = small("c4", 3, d=16, f=64, T=16, E=16)
        ref = O.forward(wl, k=0)
    elif how == "bias":
        wl = small("c2", 3, d=16, f=64, T=16, E=4)
        ref = O.forward(wl, bias=np.full(3, -1.0e30))
    else:
        wl = small("c2", 3, d=16, f=64, T=16, E=4)
        wl.x = np.zeros_like(wl.x)
        ref = O.forward(wl, bias=np.minimum(wl.bias, 0.0))
    assert np.all(ref["y"] == 0.0)
    assert np.all(ref["cnt"] == 0)
    assert np.all(ref["route"] == 0) and ref["n_dense"] == 0
    assert np.all(ref["idx"] == O.IDX_PAD)


def test_lowrank_identity_factor_equals_full_gate():
    # r = d, V = I, U = W_gate: the low-rank gate is the full gate, bit for bit
    wl = small("c2", 3, d=16, f=64, T=16, E=16)
    g_full = O.gate_preactivation(wl.x, w_gate=wl.w_gate)
    g_low = O.gate_preactivation(wl.x, u=wl.w_gate, v=np.eye(16))
    assert np.array_equal(g_full, g_low)
    # associativity: U (V x) == (U V) x to rounding
    wl3 = small("c3", 3, d=16, f=64, rank=4, T=16, E=4)
    g1 = O.gate_preactivation(wl3.x, u=wl3.u, v=wl3.v)
    g2 = wl3.x @ (wl3.u @ wl3.v).T
    assert np.allclose(g1, g2, rtol=1e-12, atol=1e-12)


def test_cut_is_strict_exact_tie_inactive():
    # dyadic toy: z hits the threshold exactly on neuron 1 -> inactive
    x = np.array([[1.0, 0.5]])
    w_gate = np.array([[1.0, 0.0], [0.5, 1.0], [2.0, 0.0], [0.0, -1.0]])
    w_up = np.ones((4, 2))
    w_down = np.eye(2, 4)
    wl = Workload(cid="toy", name="toy", d=2, f=4, rank=0, m=1, dtype="bf16", act="relu",
                  sel="thresh", T=4, E=4, k=0, seed=0, x=x, w_up=w_up, w_down=w_down,
                  w_gate=w_gate, bias=np.zeros(1), tau=np.array([1.0]))
    ref = O.forward(wl)
    # z = (1, 1, 2, -0.5): z == tau on neurons 0 and 1 -> only neuron 2 active
    assert list(np.nonzero(ref["mask"][0])[0]) == [2]
    # bias mode: z == 0 is inactive
    wl.sel, wl.tau = "bias", None
    ref = O.forward(wl, bias=np.array([-1.0]))
    assert list(np.nonzero(ref["mask"][0])[0]) == [2]


def test_threshold_below_zero_clamps_to_relu():
    wl = small("c3", 2, d=16, f=64, rank=4, T=16, E=16)
    ref = O.forward(wl, tau=np.array([-5.0, -5.0]))
    assert np.array_equal(ref["mask"], ref["z"] > 0)


# ---------------------------------------------------------------------------
# WINA: hand-computed example and Lemma 3.1 by enumeration
# ---------------------------------------------------------------------------

def _load_wina_toy():
    sec, inputs, expected = None, {}, []
    with open(os.path.join(GOLDEN, "wina_toy.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("["):
                sec = line
                continue
            parts = line.split()
            if sec == "[inputs]":
                inputs[parts[0]] = [float(p) for p in parts[1:]]
            else:
                expected.append(parts)
    x = np.array(inputs["x"]).reshape(1, 2)
    w_gate = np.array(inputs["w_gate"]).reshape(5, 2)
    w_up = np.array(inputs["w_up"]).reshape(5, 2)
    w_down = np.array(inputs["w_down_columns"]).reshape(5, 2).T      # [d, F]
    return x, w_gate, w_up, w_down, expected


def wina_toy_workload(k):
    x, w_gate, w_up, w_down, _ = _load_wina_toy()
    return Workload(cid="wina-toy", name="wina-toy", d=2, f=5, rank=0, m=1, dtype="bf16",
                    act="relu", sel="topk", T=5, E=5, k=k, seed=0, x=x, w_up=w_up,
                    w_down=w_down, w_gate=w_gate)


def test_wina_hand_example():
    _, _, _, _, expected = _load_wina_toy()
    ex = {e[0] + (e[1] if e[0] == "k" else ""): e for e in expected}
    wl = wina_toy_workload(1)
    ref = O.forward(wl)
    assert list(ref["col_norms"]) == [float(v) for v in ex["c"][1:]]
    assert list(ref["h"][0]) == [float(v) for v in ex["h"][1:]]
    assert list(ref["scores"][0]) == [float(v) for v in ex["s"][1:]]
    for k in (1, 2, 3, 4):
        e = ex["k" + str(k)]
        sel = [int(v) for v in e[e.index("sel") + 1:e.index("y")]]
        y = [float(v) for v in e[e.index("y") + 1:]]
        ref = O.forward(wina_toy_workload(k))
        assert list(ref["topk"][0]) == sel
        assert list(ref["y"][0]) == y                 # exact: every value is dyadic
    dense = O.dense_forward(wina_toy_workload(5))[0]
    wk2 = O.forward(wina_toy_workload(2))["y"][0]
    assert float(np.sum((dense - wk2) ** 2)) == 2.5
    # |h|-only selection (score without the column norm) is worse: 25 vs 2.5
    h = O.forward(wina_toy_workload(2))["h"][0]
    hsel = O.topk_lower_index(np.abs(h), 2)
    assert list(hsel) == [1, 3]
    yh = O.down_projection_sparse(h[hsel], hsel, wina_toy_workload(2).w_down)
    assert float(np.sum((dense - yh) ** 2)) == 25.0


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_wina_lemma31_optimal_for_orthogonal_columns(seed):
    """Column-orthogonal W_down: the WINA top-k set minimises ||y_dense - y_S||
    over every k-subset S (WINA page, section 3.2, Lemma 3.1)."""
    rng = np.random.default_rng(seed)
    f, d = 8, 12
    q, _ = np.linalg.qr(rng.standard_normal((d, f)))
    norms = rng.uniform(0.2, 3.0, f)
    w_down = q * norms                              # orthogonal columns, distinct norms
    h = rng.standard_normal(f)
    c = O.wina_column_norms(w_down)
    assert np.allclose(c, norms)
    s = O.wina_scores(h, c)
    y_dense = w_down @ h
    for k in range(f + 1):
        best = min(float(np.sum((y_dense - w_down[:, list(S)] @ h[list(S)]) ** 2)) if S else
                   float(np.sum(y_dense ** 2)) for S in itertools.combinations(range(f), k))
        sel = O.topk_lower_index(s, k)
        err = float(np.sum((y_dense - O.down_projection_sparse(h[sel], sel, w_down)) ** 2))
        assert err <= best * (1 + 1e-12) + 1e-15


def test_topk_tie_break_lower_index():
    s = np.array([1.0, 3.0, 3.0, 2.0, 3.0, 0.0])
    assert list(O.topk_lower_index(s, 1)) == [1]
    assert list(O.topk_lower_index(s, 2)) == [1, 2]
    assert list(O.topk_lower_index(s, 4)) == [1, 2, 3, 4]
    assert list(O.topk_lower_index(s, 0)) == []


# ---------------------------------------------------------------------------
# TwELL pack and routing
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cid,m,kw", SMALL)
def test_twell_roundtrip(cid, m, kw):
    wl = small(cid, m, **kw)
    ref = O.forward(wl)
    T, E = wl.T, wl.E
    cnt, idx, val = ref["cnt"], ref["idx"], ref["val"]
    mask, a = ref["mask"], ref["act_values"]
    assert np.array_equal(cnt.sum(axis=1), mask.sum(axis=1))
    for t in range(m):
        for j in range(wl.f // T):
            n = min(int(cnt[t, j]), E)
            ids = idx[t, j, :n].astype(int)
            assert np.all(np.diff(ids) > 0) and np.all(ids < T)
            assert np.all(idx[t, j, n:] == O.IDX_PAD)
            assert np.all(val[t, j, n:] == 0)
            cols = np.nonzero(mask[t, j * T:(j + 1) * T])[0]
            assert list(ids) == list(cols[:E])
            if wl.dtype == "f32":
                got = val[t, j, :n].astype(np.float64)
                want = a[t, j * T + ids].astype(np.float32).astype(np.float64)
            else:
                got = O.bf16_bits_to_f64(val[t, j, :n])
                want = round_bf16(a[t, j * T + ids])
            assert np.array_equal(got, want)
    route = (cnt > E).any(axis=1)
    assert np.array_equal(ref["route"].astype(bool), route)
    assert list(ref["dense_list"]) == list(np.nonzero(route)[0])


def test_routing_extremes():
    wl = small("c2", 6, d=16, f=64, T=16, E=16)
    ref = O.forward(wl, E=16)                       # E = T: nothing can overflow
    assert ref["n_dense"] == 0
    ref0 = O.forward(wl, E=0)                       # E = 0: every token with nnz > 0
    nnz = ref0["mask"].sum(axis=1)
    assert list(ref0["dense_list"]) == list(np.nonzero(nnz > 0)[0])
    assert np.array_equal(ref0["y"], ref["y"])      # routing never changes y


def test_prefill_mixture_routes_busy_tokens():
    wl = small("c5", 48, d=64, f=1024, T=256, E=32)
    ref = O.forward(wl)
    busy = wl.info["count"] > 0.15 * wl.f
    assert np.array_equal(ref["route"].astype(bool), busy)


# ---------------------------------------------------------------------------
# generator guard band, re-checked with the oracle's own pre-activations
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cid,m,kw", SMALL + [("c2", 2, {}), ("c3", 1, dict(d=512, f=1792, rank=64))])
def test_generator_guard_band(cid, m, kw):
    wl = small(cid, m, **kw)
    ref = O.forward(wl)
    z = ref["z"]
    for t in range(m):
        dl = wl.delta[t]
        if wl.sel == "topk":
            s = np.sort(ref["scores"][t])[::-1]
            k = wl.k
            if 0 < k < wl.f:
                assert s[k - 1] - s[k] >= 2.0 ** -11 * s[k - 1]
        else:
            cut = 0.0 if wl.sel == "bias" else max(wl.tau[t], 0.0)
            assert np.min(np.abs(z[t] - cut)) >= dl > 0
            assert int(ref["mask"][t].sum()) == int(wl.info["count"][t])


# ---------------------------------------------------------------------------
# input-side selection of the gate projection (WINA page, section 3.1 applied
# to the gate's input; section 二 for the |x|-only rule)
# ---------------------------------------------------------------------------

def _read_input_toy():
    sec, inp, exp = None, {}, []
    for line in open(os.path.join(GOLDEN, "input_wina_toy.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("["):
            sec = line
            continue
        parts = line.split()
        if sec == "[inputs]":
            inp[parts[0]] = [float(v) for v in parts[1:]]
        elif parts[0] in ("c", "s"):
            inp["exp_" + parts[0]] = [float(v) for v in parts[1:]]
        else:
            k = int(parts[1])
            gi = parts.index("g")
            exp.append((k, [int(v) for v in parts[3:gi]], [float(v) for v in parts[gi + 1:]]))
    return inp, exp


def test_input_wina_hand_example():
    inp, exp = _read_input_toy()
    x = np.array([inp["x"]])
    cols = np.array(inp["w_gate_columns"]).reshape(4, 2)        # column j
    w_gate = cols.T                                               # [F x d]
    c = O.input_column_norms(w_gate)
    assert list(c) == inp["exp_c"]
    s = O.input_scores(x, c)[0]
    assert list(s) == inp["exp_s"]
    for k, kept, g in exp:
        sel = O.topk_lower_index(s, k)
        assert list(sel) == kept
        assert list(O.gate_preactivation_input_sparse(x, [sel], w_gate=w_gate)[0]) == g
        # the same gate as a low-rank factorisation: V = W_gate, U = I
        gl = O.gate_preactivation_input_sparse(x, [sel], u=np.eye(2), v=w_gate)[0]
        assert list(gl) == g
    full = O.gate_preactivation(x, w_gate=w_gate)[0]
    assert list(full) == exp[-1][2]


def test_input_wina_lemma31_optimal_for_orthogonal_columns():
    """For a layer with orthogonal columns the kept input set minimises
    || W x - W_S x_S ||^2 over every k-subset, with minimum sum over dropped
    channels of (x_j c_j)^2 (WINA page, section 3.2, Lemma 3.1, on the input
    side)."""
    import itertools
    rng = np.random.default_rng(11)
    for trial in range(4):
        d, out = 6, 9
        q, _ = np.linalg.qr(rng.standard_normal((out, d)))
        w = q * rng.uniform(0.2, 3.0, size=d)                    # orthogonal columns, norms vary
        x = rng.standard_normal((1, d)) * rng.uniform(0.1, 4.0, size=d)
        c = O.input_column_norms(w)
        s = O.input_scores(x, c)[0]
        full = w @ x[0]
        for k in range(0, d + 1):
            sel = O.topk_lower_index(s, k)
            err = np.sum((full - O.gate_preactivation_input_sparse(x, [sel], w_gate=w)[0]) ** 2)
            best = min(np.sum((full - w[:, list(S)] @ x[0, list(S)]) ** 2) for S in itertools.combinations(range(d), k))
            assert err <= best * (1 + 1e-9) + 1e-12
            dropped = [j for j in range(d) if j not in set(sel.tolist())]
            assert abs(err - np.sum((x[0, dropped] * c[dropped]) ** 2)) <= 1e-9 * max(1.0, err)


def test_input_keep_all_equals_full_gate():
    for cid, kw in (("c6", dict(d=256, f=512, T=128, E=128)), ("c7", dict(d=256, f=512, rank=64, T=128, E=128))):
        wl = make_workload(cid, 3, 2, in_keep=256, **kw)
        a = O.forward(wl)
        g_full = O.gate_preactivation(wl.x, wl.w_gate, wl.u, wl.v)
        assert np.max(np.abs(a["g"] - g_full)) <= 1e-12 * np.max(np.abs(g_full))
        assert all(len(k) == 256 for k in a["in_kept"])


def test_input_equal_norms_is_magnitude_topk():
    """With every column norm equal the rule keeps the k largest |x_j|,
    ties to the lower index (section 二's hidden-state rule)."""
    rng = np.random.default_rng(5)
    d, out, k = 32, 8, 12
    w = rng.choice([-1.0, 1.0], size=(out, d))                   # every column norm exactly sqrt(8)
    x = np.round(rng.standard_normal((1, d)) * 4) / 4            # many exact ties in |x|
    s = O.input_scores(x, O.input_column_norms(w))[0]
    sel = O.topk_lower_index(s, k)
    mags = np.abs(x[0])
    want = sorted(sorted(range(d), key=lambda j: (-mags[j], j))[:k])
    assert np.array_equal(s, mags * np.sqrt(8.0))
    assert list(sel) == want


def test_input_sparse_forward_matches_bruteforce():
    """The whole forward pass with the input-side gate: dense numpy with the
    dropped input channels zeroed in the gate only (the up and down products
    use the whole x)."""
    for cid, kw in (("c6", dict(d=128, f=256, T=64, E=64)), ("c7", dict(d=128, f=256, rank=32, T=64, E=64))):
        wl = make_workload(cid, 3, 4, **kw)
        out = O.forward(wl)
        for t in range(wl.m):
            xg = np.zeros(wl.d)
            kept = out["in_kept"][t]
            xg[kept] = wl.x[t, kept]
            g = wl.w_gate @ xg if wl.w_gate is not None else wl.u @ (wl.v @ xg)
            z = g + wl.bias_per_token()[t]
            cut = 0.0 if wl.sel == "bias" else max(wl.tau[t], 0.0)
            a = np.where(z > cut, z, 0.0)
            y = wl.w_down @ (a * (wl.w_up @ wl.x[t]))
            assert np.allclose(out["y"][t], y, rtol=1e-12, atol=1e-12)
            assert len(kept) == wl.in_keep
