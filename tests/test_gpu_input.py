"""GPU parity of the input-side gate selection (config in_keep > 0): per
token the gate keeps the in_keep input channels with the largest
|x_j| * ||W[:, j]||_2 (W_gate, or V of a low-rank gate), ties to the lower
index, and reads only their weights (WINA page, section 3.1, on the gate's
input). The kept set decides the gate, so it is checked through g (the gate
error bound and the guard band), the pack (bit-exact) and y; the generator
certifies a relative gap at the in_keep-th input score."""
from __future__ import annotations

import sys

import numpy as np
import pytest

from oracle import ffn_oracle as O
from synth import Workload, make_workload
from tests.gpu_util import check_pack, check_y, host, make_ffn, sel_args, to_dev, y_to_f64
from tests.test_gpu_parity import run_full

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


CASES = [("c6", 1, {}), ("c7", 1, {}),
         ("c6", 1, dict(d=256, f=1024, T=128, E=128)),
         ("c6", 5, dict(d=512, f=2048, T=64, E=64)),
         ("c6", 40, dict(d=1024, f=2048, T=128, E=128, in_keep=300)),
         ("c6", 3, dict(d=2048, f=8192, T=128, E=128, in_keep=1)),
         ("c7", 3, dict(d=1024, f=2048, rank=128, T=128, E=128)),
         ("c7", 17, dict(d=512, f=1024, rank=64, T=64, E=64, in_keep=77)),
         ("c7", 64, dict(d=256, f=512, rank=32, T=64, E=64))]


@pytest.mark.parametrize("cid,m,kw", CASES, ids=[f"{c}-m{m}-{i}" for i, (c, m, _) in enumerate(CASES)])
def test_input_gate_parity(cid, m, kw):
    say("input gate", cid, m, kw)
    wl = make_workload(cid, m, 0, **kw)
    ffn = make_ffn(wl)
    assert ffn.forward_path(m) == "input-gate"
    run_full(wl, O.forward(wl))


@pytest.mark.parametrize("cid,kw", [("c6", dict(d=512, f=1024, T=128, E=128)),
                                    ("c7", dict(d=512, f=1024, rank=64, T=128, E=128))])
def test_input_keep_all_equals_regular_gate(cid, kw):
    """in_keep = d keeps every channel: the same pack as the regular gate and
    y within the tolerance of the same oracle."""
    say("keep all", cid, kw)
    import torch
    wl = make_workload(cid, 4, 1, in_keep=kw["d"], **kw)
    ref = O.forward(wl)
    x = to_dev(wl, wl.x)
    y1, p1 = make_ffn(wl).forward(x, **sel_args(wl))
    wl0 = make_workload(cid, 4, 1, in_keep=0, **kw)
    assert np.array_equal(wl0.x, wl.x)
    y0, p0 = make_ffn(wl0).forward(x, **sel_args(wl0))
    torch.cuda.synchronize()
    for p in (p0, p1):
        check_pack(wl, p, ref)
    check_y(y_to_f64(wl, y1)[:4], ref["y"])
    check_y(y_to_f64(wl, y0)[:4], ref["y"])


def _input_toy(k_in, lowrank):
    """The hand example of the input-side rule (tests/golden/input_wina_toy.txt)
    embedded in d = 64 input channels and F = 128 gate rows, dyadic
    throughout: scores (5, 4, 5, 3, 0, ...), a tie at 5 between channels 0
    and 2; gate rows 0 and 1 are the example's; bias -5."""
    d, f = 64, 128
    x = np.zeros((1, d))
    x[0, :4] = [1, 2, 0.5, 3]
    wg = np.zeros((f, d))
    wg[0, :4] = [3, 0, 6, 1]
    wg[1, :4] = [4, 2, 8, 0]
    wu = np.zeros((f, d))
    wu[0, 0] = 1.0
    wu[1, 1] = 0.5                                    # u = (1, 1)
    wd = np.zeros((d, f))
    wd[0, 0] = 1.0
    wd[1, 1] = 2.0
    kw = dict(cid="in-toy", name="input-toy", d=d, f=f, m=1, dtype="bf16", act="relu", sel="bias", T=64, E=64,
              k=0, seed=0, x=x, w_up=wu, w_down=wd, bias=np.array([-5.0]), delta=np.zeros(1), in_keep=k_in)
    if lowrank:
        # V = the first 64 gate rows, U = [I; 0]: the same gate through t = V x
        return Workload(rank=64, u=np.vstack([np.eye(64), np.zeros((f - 64, 64))]), v=wg[:64], **kw)
    return Workload(rank=0, w_gate=wg, **kw)


@pytest.mark.parametrize("k_in,g01", [(1, (3, 4)), (2, (6, 8)), (3, (6, 12)), (4, (9, 12)), (9, (9, 12))])
@pytest.mark.parametrize("lowrank", [False, True])
def test_input_hand_example_exact(k_in, g01, lowrank):
    say("input toy", k_in, lowrank)
    import torch
    wl = _input_toy(k_in, lowrank)
    ref = O.forward(wl)
    assert tuple(ref["g"][0, :2]) == g01
    ffn = make_ffn(wl)
    g_dbg = torch.empty((1, wl.f), dtype=torch.float32, device="cuda")
    pack = ffn.gate_pack(to_dev(wl, wl.x), g_debug=g_dbg, **sel_args(wl))
    y, pack2 = ffn.forward(to_dev(wl, wl.x), **sel_args(wl))
    torch.cuda.synchronize()
    g = g_dbg.cpu().numpy()[0].astype(np.float64)
    assert tuple(g[:2]) == g01 and np.all(g[2:] == 0.0)      # the kept set, tie to the lower index
    for p in (pack, pack2):
        assert np.array_equal(host(p.cnt)[:1], ref["cnt"])
        assert np.array_equal(host(p.idx)[:1].view(np.uint16), ref["idx"])
        assert np.array_equal(host(p.val)[:1], ref["val"])
    assert np.array_equal(host(y)[:1], O.bf16_rne_bits(ref["y"]))
