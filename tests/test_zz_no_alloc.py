"""The allocation-free forward entry point (ffn_sparse_forward_noalloc)
against ffn_sparse_forward on the same handle and inputs: the same kernels
over the library's per-GPU scratch array instead of the handle's workspace,
so pack and y must agree bit for bit, and both with the oracle. Two calls in
a row, the second with fewer tokens; configs or token counts outside the
decode sequences are refused before anything is launched."""
from __future__ import annotations

import sys

import numpy as np
import pytest

from oracle import ffn_oracle as O
from synth import make_workload
from tests.gpu_util import check_pack, check_y, host, make_ffn, sel_args, to_dev, y_to_f64

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _both(ffn, wl, m):
    import torch
    x = to_dev(wl, wl.x)[:m]
    kw = sel_args(wl)
    y1, p1 = ffn.forward(x, m=m, **kw)
    p2, y2 = ffn.new_pack(m), ffn.new_output(m)
    ffn.forward_noalloc(x, p2, y2, m=m, **kw)
    torch.cuda.synchronize()
    assert ffn.device_status() == 0
    for a, b in ((p1.cnt, p2.cnt), (p1.idx, p2.idx), (p1.val, p2.val), (p1.route, p2.route), (p1.n_dense, p2.n_dense)):
        assert np.array_equal(host(a)[: a.shape[0]], host(b)[: b.shape[0]])
    assert np.array_equal(host(y1)[:m], host(y2)[:m])
    return y2, p2


CASES = [("c3", (8, 1), dict(d=1024, f=2048, rank=128, T=128, E=16)),
         ("c2", (16, 3), dict(d=512, f=2048, T=64, E=8)),
         ("c3", (1, 1), {}),
         ("c2", (16, 1), {})]


@pytest.mark.parametrize("cid,ms,kw", CASES, ids=[f"{c}-{a}-{b}" for c, (a, b), _ in CASES])
def test_noalloc_matches_forward(cid, ms, kw):
    say("noalloc", cid, ms, kw)
    m0, m1 = ms
    wl = make_workload(cid, m0, 4, **kw)
    ffn = make_ffn(wl, max_m=m0)
    for m in (m0, m1):
        assert ffn.forward_path(m).startswith("decode")
        y, pack = _both(ffn, wl, m)
        sub = make_workload(cid, m, 4, **kw)
        ref = O.forward(sub)
        check_pack(sub, pack, ref)
        check_y(y_to_f64(sub, y)[:m], ref["y"])


def test_noalloc_refuses_other_sequences():
    say("noalloc refusals")
    import torch
    from activation_sparse_gated_amd._lib import FFN_E_UNSUPPORTED, FFNError
    wl = make_workload("c2", 24, 0, d=256, f=1024, T=128, E=16)
    ffn = make_ffn(wl)
    assert ffn.forward_path(24) == "masked-dense"
    with pytest.raises(FFNError) as e:
        ffn.forward_noalloc(to_dev(wl, wl.x), ffn.new_pack(24), ffn.new_output(24), **sel_args(wl))
    assert e.value.status == FFN_E_UNSUPPORTED
    wk = make_workload("c4", 1, 0, d=256, f=512, T=128, E=128)
    fk = make_ffn(wk)
    with pytest.raises(FFNError) as e:
        fk.forward_noalloc(to_dev(wk, wk.x), fk.new_pack(1), fk.new_output(1), **sel_args(wk))
    assert e.value.status == FFN_E_UNSUPPORTED
    torch.cuda.synchronize()
    # the refused calls launched nothing and left the handles usable
    y, pack = ffn.forward(to_dev(wl, wl.x), **sel_args(wl))
    torch.cuda.synchronize()
    check_y(y_to_f64(wl, y)[:24], O.forward(wl)["y"])
