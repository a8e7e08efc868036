"""Seeded sweep of shapes and token counts through the whole forward path
(gate_pack, updown, dense_fallback and the one-call forward) against the
oracle: model width, d_ff, TwELL tile and ELL width (down to routing most
tokens), gate rank, and 1..64 tokens, so that every kernel sequence the
library plans (one-token partial rows, split sequence, general path, top-k)
meets ragged shapes the fixed cases do not."""
from __future__ import annotations

import random

import pytest

from oracle import ffn_oracle as O
from synth import make_workload
from tests.test_gpu_parity import run_full


def _cases(n=64, seed=2024):
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        cid = rng.choice(["c2", "c2", "c3", "c3", "c3", "c4"])
        d = rng.choice([256, 512, 768, 1024, 2048, 4096] if cid != "c4" else [256, 512, 1024])
        T = rng.choice([32, 64, 128])
        f = T * rng.choice([4, 8, 16, 24, 32])
        if cid == "c4":
            f = min(f, 2048)
            f -= f % T
        E = rng.choice([T, T // 2, T // 4, max(1, T // 8)]) if cid != "c4" else T
        m = rng.choice([1, 1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 13, 16, 17, 24, 32, 64])
        kw = dict(d=d, f=f, T=T, E=E)
        if cid == "c3":
            kw["rank"] = min(rng.choice([64, 128, 256, 512]), d // 2)
        out.append((cid, m, rng.randrange(1000), kw))
    return out


CASES = _cases()


@pytest.mark.gpu
@pytest.mark.parametrize("cid,m,seed,kw", CASES, ids=[f"{c}-m{m}-s{s}-{i}" for i, (c, m, s, _) in enumerate(CASES)])
def test_sweep(cid, m, seed, kw):
    print(f"sweep {cid} m={m} seed={seed} {kw}", flush=True)
    wl = make_workload(cid, m, seed, **kw)
    run_full(wl, O.forward(wl))
