"""Seeded synthetic inputs for a mixture-of-experts layer of LoPA-gated FFNs.

The LoPA page notes that the gating carries over to mixture-of-experts
layers whose experts are FFN blocks (Mixtral, DeepSeek-V3). The shapes here
are assumptions: Mixtral-like, 8 experts of the LoPA workload's shape
(d = 4096, d_ff = 14336, rank 512, ReLU with a per-token threshold at 90%
sparsity), each token routed to 2 of them.

* expert e's weights: the LoPA workload's recipe with seed (s * 64 + e), s the
  expert seed (the token seed unless given);
* routing: per token, `topk` distinct experts uniformly at random (listed in
  ascending order), combine weights = softmax of N(0, 1) logits over the
  chosen experts, rounded to fp32;
* x_t ~ N(0, 1) rounded to bf16; for every (token, chosen expert) pair the
  threshold keeps exactly 10% of that expert's neurons, placed in a gap of
  at least 2 delta between neighbouring pre-activations (delta = 2^-13 of
  their rms); a token whose draw leaves no such gap for one of its experts is
  re-drawn (the guard band of the single-FFN workloads).

The result holds one ordinary single-FFN Workload per expert, whose tokens are
the ones routed to it in token order, so each expert can be evaluated on its
own; nothing here evaluates an expert's output.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass

import numpy as np

from .workloads import _GUARD_BF16, _SPARSITY_THRESH, _Calib, make_workload, round_bf16

_MOE_ID = 41
_S_ROUTE, _S_LOGIT, _S_XM = range(1, 4)
_MAX_ATTEMPTS = 64

MOE_CONFIGS = {
    "moe": dict(name="moe-lopa-relu-thresh-bf16-8x4096x14336-r512-top2", base="c3", experts=8, topk=2,
                ms=(1, 8)),
}


def _rng(*path) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(p) for p in path]))


@dataclass
class MoeWorkload:
    name: str
    n_experts: int
    topk: int
    m: int
    d: int
    f: int
    rank: int
    x: np.ndarray               # [m, d]
    expert_ids: np.ndarray      # [m, topk] int32, distinct and ascending per token
    weights: np.ndarray         # [m, topk] fp32 values as fp64
    tau: np.ndarray             # [m, topk] threshold of each (token, slot)
    experts: list               # Workload per expert (x = its tokens' rows)
    rows: list                  # per expert: token index of each of its rows
    slots: list                 # per expert: routing slot of each of its rows


def make_moe(m: int, *, n_experts: int = 8, topk: int = 2, seed: int = 0, base: str = "c3",
             d: int | None = None, f: int | None = None, rank: int | None = None, T: int | None = None,
             E: int | None = None, name: str = "moe", expert_seed: int | None = None) -> MoeWorkload:
    if not (1 <= topk <= n_experts):
        raise ValueError("need 1 <= topk <= n_experts")
    es = seed if expert_seed is None else expert_seed
    bases = [make_workload(base, 1, es * 64 + e, d=d, f=f, rank=rank, T=T, E=E) for e in range(n_experts)]
    b0 = bases[0]
    dd, ff = b0.d, b0.f
    k = ff - int(round(_SPARSITY_THRESH * ff))
    calibs = [_Calib(w.w_gate, w.u, w.v) for w in bases]

    rr = _rng(_MOE_ID, seed, _S_ROUTE, m)
    ids = np.stack([np.sort(rr.choice(n_experts, size=topk, replace=False)) for _ in range(m)]) \
        if m else np.zeros((0, topk), dtype=np.int64)
    lg = _rng(_MOE_ID, seed, _S_LOGIT, m).standard_normal((m, topk))
    wts = np.exp(lg - lg.max(axis=1, keepdims=True)) if m else lg
    wts = (wts / wts.sum(axis=1, keepdims=True)).astype(np.float32).astype(np.float64) if m else wts

    x = np.zeros((m, dd))
    tau = np.zeros((m, topk))
    delta = np.zeros((m, topk))
    for t in range(m):
        for a in range(_MAX_ATTEMPTS):
            xt = round_bf16(_rng(_MOE_ID, seed, _S_XM, t, a).standard_normal(dd))
            ok = True
            for s in range(topk):
                g = calibs[int(ids[t, s])].gate(xt[None, :])[0]
                dl = _GUARD_BF16 * math.sqrt(float(np.mean(g * g)))
                srt = np.sort(g)[::-1]
                if srt[k - 1] - srt[k] < 2.0 * dl:
                    ok = False
                    break
                tt = float(np.float32(0.5 * (srt[k - 1] + srt[k])))
                if np.min(np.abs(g - tt)) < dl or int(np.sum(g > tt)) != k or tt <= 0:
                    ok = False
                    break
                tau[t, s] = tt
                delta[t, s] = dl
            if ok:
                x[t] = xt
                break
        else:
            raise RuntimeError(f"no certified draw for token {t}")

    experts, rows, slots = [], [], []
    for e in range(n_experts):
        r_e, s_e = np.nonzero(ids == e)
        order = np.argsort(r_e, kind="stable")
        r_e, s_e = r_e[order], s_e[order]
        me = int(r_e.size)
        wl = dataclasses.replace(
            bases[e], m=me, x=x[r_e].copy() if me else np.zeros((0, dd)), tau=tau[r_e, s_e].copy(),
            bias=np.zeros(me), delta=delta[r_e, s_e].copy(), attempts=np.zeros(me, dtype=np.int64),
            info={"target_count": np.full(me, k), "count": np.full(me, k), "certified": True})
        experts.append(wl)
        rows.append(r_e.astype(np.int64))
        slots.append(s_e.astype(np.int64))
    return MoeWorkload(name=name, n_experts=n_experts, topk=topk, m=m, d=dd, f=ff, rank=b0.rank, x=x,
                       expert_ids=ids.astype(np.int32), weights=wts, tau=tau, experts=experts, rows=rows,
                       slots=slots)


def make_moe_config(cid: str, m: int | None = None, seed: int = 0, **kw) -> MoeWorkload:
    cfg = MOE_CONFIGS[cid]
    mm = cfg["ms"][0] if m is None else m
    kw.setdefault("n_experts", cfg["experts"])
    kw.setdefault("topk", cfg["topk"])
    return make_moe(mm, seed=seed, base=cfg["base"], name=cfg["name"], **kw)
