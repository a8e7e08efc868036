"""GPU parity of the decode kernel sequence (bf16, bias / threshold gate,
1..8 tokens): gate sub-tiles with look-back, the up products in the gate
workgroups, the column-chunk down kernel. Every case asserts that forward()
takes that sequence, then checks the pack (bit-exact), the gate against the
guard band and y against the oracle, through both the standalone entry points
and forward()."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest

from oracle import ffn_oracle as O
from synth import make_workload
from tests.gpu_util import check_pack, check_y, host, make_ffn, sel_args, to_dev, y_to_f64
from tests.test_gpu_parity import run_full

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


# (workload, tokens, overrides): gate rows per workgroup R = NW * IPW / P with
# P = pieces of 512 per gate row, NW = 16 waves and IPW up to 8 for one token,
# 8 waves and IPW up to 4 otherwise; the comment gives (P, R, sub-tiles per
# TwELL tile)
DECODE = [
    ("c2", 1, dict(d=256, f=1024, T=128, E=16)),          # P1 R64 Q2
    ("c2", 3, dict(d=512, f=2048, T=64, E=8)),            # P1 R32 Q2
    ("c2", 8, dict(d=1024, f=2048, T=128, E=16)),         # P2 R16 Q8
    ("c2", 2, dict(d=2048, f=4096, T=128, E=64)),         # P4 R8  Q16
    ("c2", 4, dict(d=4096, f=2048, T=64, E=8)),           # P8 R4  Q16
    ("c2", 1, dict(d=4096, f=2048, T=64, E=8)),           # P8 R16 Q4
    ("c2", 1, dict(d=2048, f=4096, T=128, E=64)),         # P4 R32 Q4
    ("c2", 4, dict(d=192, f=768, T=32, E=4)),             # P1 R32 Q1, partial piece
    ("c2", 7, dict(d=256, f=1024, T=16, E=16)),           # P1 R16 Q1
    ("c3", 1, dict(d=512, f=1792, rank=64, T=128, E=16)),
    ("c3", 6, dict(d=1024, f=2048, rank=128, T=128, E=8)),
    ("c3", 8, dict(d=2048, f=2048, rank=256, T=64, E=4)),
    ("c3", 2, dict(d=4096, f=1024, rank=512, T=128, E=64)),
    ("c3", 5, dict(d=1024, f=2048, rank=512, T=128, E=16)),  # matrix-core gate (R32, K512), ragged M
    ("c3", 7, dict(d=512, f=4096, rank=512, T=64, E=8)),     # matrix-core gate, two sub-tiles per tile
    ("c2", 16, dict(d=2048, f=4096, T=128, E=64)),           # 9..16 tokens: split sequence, two tokens a wave
    ("c2", 11, dict(d=512, f=2048, T=64, E=8)),
    ("c3", 13, dict(d=1024, f=2048, rank=512, T=128, E=16)),
    ("c3", 16, dict(d=4096, f=2048, rank=512, T=128, E=16)),  # 16 tokens' x at d = 4096 in the up kernel's LDS
    ("c3", 12, dict(d=4096, f=4096, rank=512, T=64, E=8)),
]


@pytest.mark.parametrize("cid,m,kw", DECODE, ids=[f"{c}-m{m}-{i}" for i, (c, m, _) in enumerate(DECODE)])
def test_decode_parity(cid, m, kw):
    say("decode", cid, m, kw)
    wl = make_workload(cid, m, 0, **kw)
    ffn = make_ffn(wl)
    assert ffn.forward_path(m).startswith("decode")
    ref = O.forward(wl)
    run_full(wl, ref)


@pytest.mark.parametrize("E", [0, 2, 16])
def test_decode_routed_tokens(E):
    """Tokens whose tiles overflow E keep every active neuron in the hidden
    list: y is complete, and route / dense_list still mark them."""
    say("decode routed E", E)
    wl = make_workload("c2", 6, 1, d=256, f=1024, T=16, E=16)
    ref = O.forward(wl, E=E)
    if E == 0:
        assert ref["n_dense"] == int((ref["mask"].sum(axis=1) > 0).sum())
    assert make_ffn(wl, E=E).forward_path(6).startswith("decode")
    run_full(wl, ref, E=E)


MODES = (({"FFN_SPARSE_DEC_MODE": "1"}, "decode-chunk"), ({"FFN_SPARSE_DEC_MODE": "2"}, "decode-part"),
         ({"FFN_SPARSE_DEC_MODE": "3"}, "decode-split"), ({"FFN_SPARSE_NO_DECODE": "1"}, "general"))


@pytest.mark.parametrize("cid,m,kw", [("c3", 1, dict(d=1024, f=2048, rank=128, T=128, E=16)),
                                      ("c3", 2, dict(d=1024, f=2048, rank=128, T=128, E=16)),
                                      ("c3", 4, dict(d=1024, f=2048, rank=128, T=128, E=16)),
                                      ("c3", 8, dict(d=1024, f=2048, rank=128, T=128, E=16)),
                                      ("c2", 3, dict(d=2048, f=4096, T=128, E=4)),
                                      ("c2", 1, dict(d=192, f=768, T=32, E=4)),
                                      ("c2", 4, dict(d=4096, f=1024, T=64, E=8))])
def test_decode_modes_and_general_agree(cid, m, kw):
    """The three decode down-projection organisations and the general
    sequence (all forced through the tuning switches) give the same pack and y
    within the parity tolerance; each is bitwise reproducible."""
    say("decode modes vs general", cid, m, kw)
    import torch
    wl = make_workload(cid, m, 2, **kw)
    ref = O.forward(wl)
    x = to_dev(wl, wl.x)
    outs = []
    for env, path in MODES:
        os.environ.update(env)
        try:
            ffn = make_ffn(wl)
        finally:
            for k in env:
                os.environ.pop(k, None)
        if path == "decode-split" and (wl.d % 256 or wl.d > 4096):
            path = "decode-chunk"        # the split sequence needs d a multiple of 256, at most 4096
        assert ffn.forward_path(wl.m) == path
        y, pack = ffn.forward(x, **sel_args(wl))
        torch.cuda.synchronize()
        check_pack(wl, pack, ref)
        check_y(y_to_f64(wl, y)[: wl.m], ref["y"])
        y_again, _ = ffn.forward(x, **sel_args(wl))
        torch.cuda.synchronize()
        assert np.array_equal(host(y_again), host(y))
        outs.append((host(pack.cnt).copy(), host(pack.idx).copy()))
    for o in outs[1:]:
        assert np.array_equal(outs[0][0], o[0]) and np.array_equal(outs[0][1], o[1])


def test_decode_all_masked_and_single_token_repeat():
    """All-masked tokens give exact zero rows; repeated calls on one handle
    (look-back epochs advancing) give identical results."""
    say("decode masked / repeat")
    import torch
    from tests.gpu_util import f32_dev
    wl = make_workload("c2", 3, 0, d=512, f=2048, T=128, E=16)
    ffn = make_ffn(wl)
    x = to_dev(wl, wl.x)
    bias = wl.bias.copy()
    bias[1] = -1e30
    y, pack = ffn.forward(x, bias=f32_dev(bias))
    torch.cuda.synchronize()
    ref = O.forward(wl, bias=bias)
    check_pack(wl, pack, ref)
    assert np.all(host(pack.cnt)[1] == 0)
    yy = y_to_f64(wl, y)
    assert np.all(yy[1] == 0.0)
    check_y(yy[:3], ref["y"])
    first = host(y).copy()
    for _ in range(5):
        y, pack = ffn.forward(x, bias=f32_dev(bias))
        torch.cuda.synchronize()
        assert np.array_equal(host(y), first)


@pytest.mark.parametrize("m,kw", [(1, dict(d=512, f=1024, T=128, E=128)),
                                  (1, dict(d=1024, f=2816, T=128, E=128)),
                                  (3, dict(d=512, f=1024, T=128, E=128)),
                                  (1, dict(d=192, f=768, T=64, E=64))])
def test_topk_down_organisations(m, kw):
    """Top-k selection's down product through the one-token list kernel (one
    token), the dense product of the masked h rows (several tokens, or a shape
    the list kernel does not take) and the per-token TwELL kernel (forced by
    the tuning switch) all match the oracle, pack and y, reproducibly."""
    say("topk down", m, kw)
    import torch
    wl = make_workload("c4", m, 3, **kw)
    ref = O.forward(wl)
    x = to_dev(wl, wl.x)
    ys = []
    for env in ({}, {"FFN_SPARSE_NO_TOPK_DOWN": "1"}):
        os.environ.update(env)
        try:
            ffn = make_ffn(wl)
        finally:
            for k in env:
                os.environ.pop(k, None)
        want = "general" if env else ("topk-list" if m == 1 and wl.d % 256 == 0 else "topk-masked-dense")
        assert ffn.forward_path(wl.m) == want
        y, pack = ffn.forward(x, **sel_args(wl))
        torch.cuda.synchronize()
        check_pack(wl, pack, ref)
        check_y(y_to_f64(wl, y)[: wl.m], ref["y"])
        y2, _ = ffn.forward(x, **sel_args(wl))
        torch.cuda.synchronize()
        assert np.array_equal(host(y2), host(y))
        ys.append(host(y)[: wl.m].copy())

