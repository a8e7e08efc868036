"""GPU parity of the mixture-of-experts layer over sparse LoPA FFN experts.

LoPA page, "Model Casting and Quality at 90% Sparsity": the gating carries
over to MoE layers whose experts are FFN blocks. Each expert runs the
library's own sparse forward pass on its tokens; the layer output is the
routing-weighted sum per token, compared with the oracle per token within
the workload's relative L2 bound.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

from oracle import ffn_oracle as O
from synth.moe import make_moe, make_moe_config
from tests.gpu_util import check_y, f32_dev, make_ffn, to_dev

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def run_moe(mw, max_m=None):
    import torch
    from activation_sparse_gated_amd import moe_forward
    experts = [make_ffn(wl, max_m=max(mw.m, 1) if max_m is None else max_m) for wl in mw.experts]
    x = to_dev(mw.experts[0], mw.x)
    tau = f32_dev(mw.tau)
    y = moe_forward(experts, x, mw.expert_ids, mw.weights, tau=tau)
    torch.cuda.synchronize()
    return experts, x, tau, y[:mw.m].float().cpu().numpy().astype(np.float64)


SMALL = dict(d=256, f=1024, rank=32, T=64, E=64)
CASES = [(6, 4, 2, 0), (9, 3, 3, 1), (5, 1, 1, 2), (16, 8, 2, 3), (40, 4, 1, 4)]


# experts of rank 512 (the shape the grouped split sequence is built for):
# 2..8 tokens per expert run as one group, one-token experts as another, and
# experts with more tokens alone
LR512 = dict(d=1024, f=2048, rank=512, T=128, E=64)
CASES512 = [(8, 8, 2, 5), (12, 4, 2, 6), (20, 4, 2, 7), (3, 8, 2, 8)]


@pytest.mark.parametrize("m,ne,k,seed", CASES512, ids=[f"r512-m{c[0]}-e{c[1]}-top{c[2]}" for c in CASES512])
def test_moe_grouped_sequences(m, ne, k, seed):
    say("moe grouped", m, ne, k, seed)
    mw = make_moe(m, n_experts=ne, topk=k, seed=seed, **LR512)
    counts = [wl.m for wl in mw.experts]
    say("tokens per expert", counts)
    _, _, _, y = run_moe(mw)
    check_y(y, O.moe_forward(mw)["y"])


@pytest.mark.parametrize("m,ne,k,seed", CASES, ids=[f"m{c[0]}-e{c[1]}-top{c[2]}" for c in CASES])
def test_moe_parity_small(m, ne, k, seed):
    say("moe small", m, ne, k, seed)
    mw = make_moe(m, n_experts=ne, topk=k, seed=seed, **SMALL)
    _, _, _, y = run_moe(mw)
    check_y(y, O.moe_forward(mw)["y"])


def test_moe_argument_errors():
    import torch
    from activation_sparse_gated_amd import FFNError, moe_forward
    say("moe errors")
    mw = make_moe(4, n_experts=3, topk=2, seed=5, **SMALL)
    experts = [make_ffn(wl, max_m=3) for wl in mw.experts]   # an expert takes at most 3 tokens
    x = to_dev(mw.experts[0], mw.x)
    tau = f32_dev(mw.tau)
    ok_ids = np.array([[0, 1], [1, 2], [0, 2], [0, 1]], dtype=np.int32)   # 3, 3 and 2 tokens
    moe_forward(experts, x, ok_ids, mw.weights, tau=tau)
    dup = ok_ids.copy()
    dup[0, 1] = dup[0, 0]                                  # one expert twice for a token
    with pytest.raises(FFNError):
        moe_forward(experts, x, dup, mw.weights, tau=tau)
    crowded = np.array([[0, 1]] * 4, dtype=np.int32)       # expert 0 gets 4 tokens > max_m
    with pytest.raises(FFNError):
        moe_forward(experts, x, crowded, mw.weights, tau=tau)
    with pytest.raises(FFNError):                          # a threshold config needs tau
        moe_forward(experts, x, ok_ids, mw.weights)
    torch.cuda.synchronize()


@pytest.mark.parametrize("m,ne", [(1, 2), (4, 4), (8, 8)])   # (8, 8): the timed 8-token configuration
def test_moe_full_size(m, ne):
    """Experts of the LoPA shape (d = 4096, d_ff = 14336, rank 512), top-2."""
    say("moe full size", m, ne)
    mw = make_moe_config("moe", m=m, seed=0, n_experts=ne)
    _, _, _, y = run_moe(mw)
    check_y(y, O.moe_forward(mw)["y"])
