"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Bit-exact: masks / top-k sets (via the pack's cnt and idx), route,
dense_list. Pack values: within 1 bf16 ulp. y: per-token relative L2 within
5e-3. The GPU gate is also checked against the certified guard band.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

from oracle import ffn_oracle as O
from synth import Workload, make_workload
from tests.gpu_util import (check_gate_band, check_pack, check_scores, check_y, f32_dev, host, make_ffn, sel_args,
                            to_dev, y_to_f64)

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def run_full(wl, ref, *, E=None, check_band=True):
    import torch
    ffn = make_ffn(wl, E=E)
    x = to_dev(wl, wl.x)
    g_dbg = torch.empty((wl.m, wl.f), dtype=torch.float32, device="cuda")
    s_dbg = torch.empty((wl.m, wl.f), dtype=torch.float32, device="cuda") if wl.sel == "topk" else None
    kw = sel_args(wl)
    pack = ffn.gate_pack(x, g_debug=g_dbg, s_debug=s_dbg, **kw)
    torch.cuda.synchronize()
    if check_band and wl.sel != "topk":
        check_gate_band(wl, g_dbg.cpu().numpy(), ref)
    if wl.sel == "topk":
        check_scores(wl, s_dbg.cpu().numpy(), ref)
    check_pack(wl, pack, ref, E=E)
    y = ffn.updown(x, pack)
    ffn.dense_fallback(x, pack, y, **kw)
    torch.cuda.synchronize()
    worst = check_y(y_to_f64(wl, y)[: wl.m], ref["y"])
    # the one-call forward: same pack. On the general path non-routed rows are
    # bit-identical (same sparse kernel); the decode and top-k sequences sum in
    # another order, so there only the oracle comparison applies
    y2, pack2 = ffn.forward(x, **kw)
    torch.cuda.synchronize()
    check_pack(wl, pack2, ref, E=E)
    if ffn.forward_path(wl.m) == "general":
        keep = ref["route"][: wl.m] == 0
        assert np.array_equal(host(y2)[: wl.m][keep], host(y)[: wl.m][keep])
    check_y(y_to_f64(wl, y2)[: wl.m], ref["y"])
    if (wl.E if E is None else E) > 0:
        assert np.array_equal(host(pack2.idx)[: wl.m], host(pack.idx)[: wl.m])
    return worst


# ---------------------------------------------------------------------------
# reduced sizes: several tiles, ragged token counts, every mode
# ---------------------------------------------------------------------------

REDUCED = [
    ("c1", 4, {}),                                                  # the tiny fp32 workload itself
    ("c1", 5, dict(d=128, f=512, T=32, E=8)),
    ("c2", 5, dict(d=256, f=1024, T=128, E=16)),
    ("c2", 19, dict(d=512, f=2048, T=64, E=8)),
    ("c3", 3, dict(d=512, f=1792, rank=64, T=128, E=16)),
    ("c3", 37, dict(d=256, f=1024, rank=32, T=64, E=8)),
    ("c4", 3, dict(d=512, f=1024, T=128, E=128)),
    ("c4", 18, dict(d=256, f=768, T=64, E=64)),
    # top-k workgroups per token: 3 tiles (3 workgroups), 17 tiles over 16,
    # 2 workgroups a token, 1 workgroup a token
    ("c4", 1, dict(d=256, f=384, T=128, E=128)),
    ("c4", 1, dict(d=256, f=1088, T=64, E=64)),
    ("c4", 100, dict(d=256, f=640, T=64, E=64)),
    ("c4", 300, dict(d=128, f=512, T=64, E=64)),
    # the general path past two workgroups per CU: eight XCD-aligned tile
    # groups (90 tokens), then four (110 tokens)
    ("c3", 90, dict(d=512, f=2048, rank=64, T=128, E=64)),
    ("c3", 110, dict(d=512, f=2048, rank=64, T=128, E=64)),
    ("c5", 67, dict(d=256, f=2048, T=256, E=32)),
    ("c5", 40, dict(d=128, f=1024, T=1024, E=128)),
]


@pytest.mark.parametrize("cid,m,kw", REDUCED, ids=[f"{c}-m{m}-{i}" for i, (c, m, _) in enumerate(REDUCED)])
def test_reduced(cid, m, kw):
    say("reduced", cid, m, kw)
    wl = make_workload(cid, m, 0, **kw)
    ref = O.forward(wl)
    run_full(wl, ref)


# 17..127 tokens run the masked dense sequence; the general sequence (sparse
# up + down over the pack, dense backup of routed tokens) is kept reachable
# by a path switch and must agree with it and with the oracle
MIDSIZE = [
    ("c2", 19, dict(d=512, f=2048, T=64, E=8)),
    ("c3", 37, dict(d=256, f=1024, rank=32, T=64, E=8)),
    ("c3", 64, dict(d=1024, f=4096, rank=128, T=128, E=64)),
    ("c5", 67, dict(d=256, f=2048, T=256, E=32)),
    # the prefill shape at 100 tokens: two token blocks; forced onto the
    # general path, the routed tokens' dense down product runs on the skinny
    # GEMM with K split four ways, a device-side token count and scattered rows
    ("c5", 100, dict(T=1024, E=128)),
    # ELL width 0 (every token with an active neuron is routed) and TwELL
    # tiles narrower than a wave
    ("c2", 20, dict(d=256, f=1024, T=32, E=0)),
    # 72 TwELL tiles, more than the XCD-sliced pair holds: the masked dense
    # sequence up to 256 tokens, three token blocks
    ("c3", 160, dict(d=512, f=9216, rank=64, T=128, E=64)),
]


@pytest.mark.parametrize("cid,m,kw", MIDSIZE, ids=[f"{c}-m{m}" for c, m, _ in MIDSIZE])
def test_masked_dense_and_general_agree(cid, m, kw):
    say("masked dense vs general", cid, m, kw)
    import os

    import torch
    wl = make_workload(cid, m, 1, **kw)
    ref = O.forward(wl)
    x = to_dev(wl, wl.x)
    outs = []
    for env, path in (({}, "masked-dense"), ({"FFN_SPARSE_NO_MASKED_DENSE": "1"}, "general")):
        os.environ.update(env)
        try:
            ffn = make_ffn(wl)
        finally:
            for k in env:
                os.environ.pop(k, None)
        assert ffn.forward_path(wl.m) == path
        y, pack = ffn.forward(x, **sel_args(wl))
        torch.cuda.synchronize()
        check_pack(wl, pack, ref)
        check_y(y_to_f64(wl, y)[: wl.m], ref["y"])
        y_again, _ = ffn.forward(x, **sel_args(wl))
        torch.cuda.synchronize()
        assert np.array_equal(host(y_again), host(y))
        # the first E slots of each tile are defined (E = 0 leaves none)
        outs.append((host(pack.cnt).copy(), host(pack.idx)[..., : wl.E].copy(), host(pack.route).copy()))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("E", [0, 4, 8, 64])
def test_tiny_fp32_ell_widths(E):
    say("c1 E", E)
    wl = make_workload("c1", 4, 0)
    ref = O.forward(wl, E=E)
    run_full(wl, ref, E=E)


@pytest.mark.parametrize("E", [0, 16])
def test_bf16_all_routed_and_none(E):
    say("c2-reduced E", E)
    wl = make_workload("c2", 9, 1, d=256, f=1024, T=16, E=16)
    ref = O.forward(wl, E=E)
    if E == 0:
        assert ref["n_dense"] == int((ref["mask"].sum(axis=1) > 0).sum())
    run_full(wl, ref, E=E)


def test_lowrank_reduced_out_major_and_neuron_major():
    say("c3 wdown layouts")
    import torch
    wl = make_workload("c3", 6, 2, d=256, f=1024, rank=64, T=128, E=8)
    ref = O.forward(wl)
    ys = []
    for om in (True, False):
        ffn = make_ffn(wl, wdown_out_major=om)
        y, pack = ffn.forward(to_dev(wl, wl.x), **sel_args(wl))
        torch.cuda.synchronize()
        check_pack(wl, pack, ref)
        check_y(y_to_f64(wl, y)[: wl.m], ref["y"])
        ys.append(host(y))
    assert np.array_equal(ys[0], ys[1])


# ---------------------------------------------------------------------------
# the workloads at full size
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cid,m", [("c2", 1), ("c2", 16), ("c3", 1), ("c3", 8), ("c4", 1), ("c5", 4096)])
def test_full_size(cid, m):
    say("full", cid, m)
    wl = make_workload(cid, m, 0)
    ref = O.forward(wl)
    run_full(wl, ref)


@pytest.mark.parametrize("cid,m", [("c3", 64), ("c4", 32)])
def test_full_size_batched(cid, m):
    say("full", cid, m)
    wl = make_workload(cid, m, 0)
    ref = O.forward(wl)
    run_full(wl, ref)


# ---------------------------------------------------------------------------
# special cases and invariants on the GPU
# ---------------------------------------------------------------------------

def _wina_toy_padded(k):
    """The hand-computed WINA example embedded in d = 64, F = 128 (T = E = 64)
    with zero padding: the padded neurons score 0 and the padded inputs are 0."""
    x = np.zeros((1, 64)); x[0, :2] = [1, 2]
    wg = np.zeros((128, 64)); wu = np.zeros((128, 64)); wd = np.zeros((64, 128))
    wg[:5, 0] = [1, 1, 1, 1, -1]
    wu[:5, 0] = [0.5, -1.25, 0.25, 3, 7]
    cols = [(3, 4), (0, 2), (6, 8), (1, 0), (0, 1)]
    for i, (a, b) in enumerate(cols):
        wd[0, i], wd[1, i] = a, b
    return Workload(cid="wina-toy", name="wina-toy", d=64, f=128, rank=0, m=1, dtype="bf16", act="relu",
                    sel="topk", T=64, E=64, k=k, seed=0, x=x, w_up=wu, w_down=wd, w_gate=wg,
                    delta=np.zeros(1))


@pytest.mark.parametrize("k,sel,y", [(1, [3], (3, 0)), (2, [0, 3], (4.5, 2)), (3, [0, 1, 3], (4.5, -0.5)),
                                     (4, [0, 1, 2, 3], (6, 1.5))])
def test_wina_hand_example_exact(k, sel, y):
    say("wina toy k", k)
    import torch
    wl = _wina_toy_padded(k)
    ffn = make_ffn(wl)
    yy, pack = ffn.forward(to_dev(wl, wl.x), k=k)
    torch.cuda.synchronize()
    cnt = host(pack.cnt)[0]
    idx = host(pack.idx)[0].view(np.uint16)
    assert cnt[0] == k and cnt[1] == 0
    assert list(idx[0, :k]) == sel
    out = y_to_f64(wl, yy)[0]
    assert list(out[:2]) == list(y) and np.all(out[2:] == 0)      # exact, y included


def test_all_masked_exact_zero():
    say("all masked")
    import torch
    wl = make_workload("c2", 5, 0, d=256, f=1024, T=128, E=16)
    ffn = make_ffn(wl)
    y, pack = ffn.forward(to_dev(wl, wl.x), bias=f32_dev(np.full(5, -1e30)))
    torch.cuda.synchronize()
    assert np.all(host(pack.cnt) == 0)
    assert int(host(pack.n_dense)[0]) == 0
    assert np.all(y_to_f64(wl, y) == 0.0)


@pytest.mark.parametrize("k", [0, 1024])
def test_topk_extremes(k):
    say("topk k", k)
    import torch
    wl = make_workload("c4", 3, 0, d=256, f=1024, T=128, E=128, k=k)
    ref = O.forward(wl, k=k)
    ffn = make_ffn(wl)
    y, pack = ffn.forward(to_dev(wl, wl.x), k=k)
    torch.cuda.synchronize()
    check_pack(wl, pack, ref)
    check_y(y_to_f64(wl, y)[:3], ref["y"])
    if k == 1024:
        check_y(y_to_f64(wl, y)[:3], O.dense_forward(wl))


def test_zero_tokens():
    say("m = 0")
    import torch
    wl = make_workload("c2", 2, 0, d=256, f=1024, T=128, E=16)
    ffn = make_ffn(wl)
    pack = ffn.new_pack(1)
    pack.n_dense.fill_(7)
    ffn.forward(to_dev(wl, wl.x), m=0, pack=pack, **sel_args(wl))
    torch.cuda.synchronize()
    assert int(host(pack.n_dense)[0]) == 0


def test_lowrank_identity_gate_equals_full_gate():
    say("low-rank identity")
    import torch
    full = make_workload("c2", 4, 3, d=256, f=1024, T=128, E=16)
    low = Workload(cid="id", name="id", d=256, f=1024, rank=256, m=4, dtype="bf16", act="relu",
                   sel="bias", T=128, E=16, k=0, seed=3, x=full.x, w_up=full.w_up, w_down=full.w_down,
                   u=full.w_gate, v=np.eye(256), bias=full.bias, delta=full.delta)
    ref = O.forward(full)
    packs = []
    for wl in (full, low):
        ffn = make_ffn(wl)
        y, pack = ffn.forward(to_dev(wl, wl.x), **sel_args(wl))
        torch.cuda.synchronize()
        check_pack(wl, pack, ref)
        check_y(y_to_f64(wl, y)[:4], ref["y"])
        packs.append(pack)
    assert np.array_equal(host(packs[0].cnt), host(packs[1].cnt))
    assert np.array_equal(host(packs[0].idx), host(packs[1].idx))


def test_run_to_run_bitwise():
    say("determinism")
    import torch
    wl = make_workload("c3", 8, 1, d=512, f=1792, rank=64, T=128, E=16)
    ffn = make_ffn(wl)
    x = to_dev(wl, wl.x)
    outs = []
    for _ in range(3):
        y, pack = ffn.forward(x, **sel_args(wl))
        torch.cuda.synchronize()
        outs.append((host(y).copy(), host(pack.val).copy(), host(pack.idx).copy()))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b)


@pytest.mark.parametrize("cid,m,kw", [("c2", 7, dict(d=256, f=1024, T=128, E=16)),
                                      ("c3", 5, dict(d=256, f=1024, rank=32, T=128, E=16)),
                                      ("c4", 4, dict(d=256, f=768, T=128, E=128)),
                                      ("c1", 4, {})])
def test_dense_forward(cid, m, kw):
    say("dense", cid, m)
    import torch
    wl = make_workload(cid, m, 0, **kw)
    ffn = make_ffn(wl)
    kw2 = sel_args(wl)
    kw2.pop("k", None)
    y = ffn.dense_forward(to_dev(wl, wl.x), **kw2)
    torch.cuda.synchronize()
    check_y(y_to_f64(wl, y)[:m], O.dense_forward(wl))


def test_graph_replay_matches_eager():
    say("graph replay")
    import torch
    wl = make_workload("c3", 4, 0, d=512, f=1792, rank=64, T=128, E=16)
    ffn = make_ffn(wl)
    x = to_dev(wl, wl.x)
    kw = sel_args(wl)
    pack = ffn.new_pack(wl.m)
    y = ffn.new_output(wl.m)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ffn.forward(x, pack=pack, y=y, **kw)
    torch.cuda.synchronize()
    eager = host(y).copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ffn.forward(x, pack=pack, y=y, **kw)
    for _ in range(4):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(y), eager)
        ffn.forward(x, pack=pack, y=y, **kw)      # eager work between replays
        torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# prefill-shaped GEMMs (128+ tokens): several 128-token tiles, a ragged last
# tile, the dense backup on a gathered token list, the dense baseline
# ---------------------------------------------------------------------------

PREFILL = [
    ("c5", 300, dict(d=256, f=2048, T=256, E=32)),
    ("c2", 200, dict(d=512, f=1024, T=128, E=16)),
    ("c4", 160, dict(d=256, f=768, T=128, E=128)),
    ("c5", 261, dict(d=1024, f=2048, T=256, E=32)),
    ("c2", 300, dict(d=512, f=4096, T=64, E=8)),
    ("c3", 150, dict(d=512, f=1024, rank=64, T=128, E=16)),
]


@pytest.mark.parametrize("cid,m,kw", PREFILL, ids=[f"{c}-m{m}" for c, m, _ in PREFILL])
def test_prefill_shapes(cid, m, kw):
    say("prefill", cid, m, kw)
    import os
    import torch
    wl = make_workload(cid, m, 0, **kw)
    ref = O.forward(wl)
    run_full(wl, ref)
    # the same pack and y (within tolerance) without the prefill-shaped kernel
    os.environ["FFN_SPARSE_NO_PREFILL_GEMM"] = "1"
    try:
        ffn = make_ffn(wl)
    finally:
        os.environ.pop("FFN_SPARSE_NO_PREFILL_GEMM", None)
    y2, pack2 = ffn.forward(to_dev(wl, wl.x), **sel_args(wl))
    torch.cuda.synchronize()
    check_pack(wl, pack2, ref)
    check_y(y_to_f64(wl, y2)[: wl.m], ref["y"])
    if wl.sel != "topk":
        kw2 = sel_args(wl)
        kw2.pop("k", None)
        yd = make_ffn(wl).dense_forward(to_dev(wl, wl.x), **kw2)
        torch.cuda.synchronize()
        check_y(y_to_f64(wl, yd)[: wl.m], O.dense_forward(wl))


@pytest.mark.parametrize("cid,m,kw", [("c5", 261, dict(d=1024, f=2048, T=256, E=32)),
                                      ("c2", 300, dict(d=512, f=4096, T=64, E=8))])
def test_prefill_xcd_pair_vs_per_token_kernel(cid, m, kw):
    """The XCD-sliced up / down pair and the per-token sparse kernel (forced by
    the tuning switch) give the same pack and y within the parity tolerance
    against the oracle; the pair is bitwise reproducible."""
    say("prefill xcd vs per-token", cid, m, kw)
    import os
    import torch
    wl = make_workload(cid, m, 1, **kw)
    ref = O.forward(wl)
    x = to_dev(wl, wl.x)
    outs = []
    for env in ({}, {"FFN_SPARSE_NO_XCD": "1"}):
        os.environ.update(env)
        try:
            ffn = make_ffn(wl)
        finally:
            for k in env:
                os.environ.pop(k, None)
        y, pack = ffn.forward(x, **sel_args(wl))
        torch.cuda.synchronize()
        check_pack(wl, pack, ref)
        check_y(y_to_f64(wl, y)[: wl.m], ref["y"])
        y2, _ = ffn.forward(x, **sel_args(wl))
        torch.cuda.synchronize()
        assert np.array_equal(host(y2), host(y))
        outs.append(host(y)[: wl.m].copy())
