"""GPU parity of the sparse FFN's backward pass against the oracle.

Sparser/Faster/Lighter page, "Hybrid 應對非均勻稀疏": training with the
compact format for most tokens and a dense backup for busy ones. The GPU
pass takes the forward pass's pack (activations a as stored: bf16 in bf16
configs, a relative rounding of 2^-9 that enters du = dh a) and recomputes
routed tokens' gate rows. Checked: dx per token, and every gradient row of
W_up, W_gate and W_down (neuron-major) within the workload's relative L2
bound of 5e-3; rows of neurons no token activates stay exactly zero; a
second call adds the same values again (exact doubling). At 4096 tokens the
oracle evaluates a sample of tokens (routed ones among them) and neurons on
its own (`backward_sampled`). From 512 tokens dx
is a bf16 GEMM of the dense (du | dz) rows: du and dz rounded to bf16 add a
relative error of about 2^-9 / sqrt(3) per token, inside the same bound.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

from oracle import ffn_oracle as O
from synth import draw_dy, make_workload
from tests.gpu_util import check_y, make_ffn, sel_args, to_dev, y_to_f64

pytestmark = pytest.mark.gpu
TOL = 5e-3


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def check_rows(got, ref, what):
    for i in range(ref.shape[0]):
        nr = np.linalg.norm(ref[i])
        if nr == 0.0:
            assert np.all(got[i] == 0.0), f"{what} row {i}: must stay zero"
            continue
        rel = np.linalg.norm(got[i] - ref[i]) / nr
        assert rel <= TOL, f"{what} row {i}: rel L2 {rel:.3e}"


CASES = [("c1", 4, {}), ("c2", 5, dict(d=256, f=1024)), ("c2", 70, dict(d=256, f=1024)),
         ("c5", 40, dict(d=256, f=1024, T=256, E=16)), ("c2", 16, {}), ("c5", 200, dict(d=512, f=2048)),
         ("c5", 256, {}),                                  # full width: d 2048, d_ff 8192, T 1024, E 128
         # 512+ tokens: dx as a matrix-core GEMM of the dense (du | dz) rows
         ("c2", 520, dict(d=256, f=1024)), ("c5", 600, dict(d=512, f=2048, T=256, E=32)),
         ("c5", 4096, {})]                                 # the timed configuration: 4096 tokens, full width


@pytest.mark.parametrize("cid,m,kw", CASES, ids=[f"{c}-m{m}-{i}" for i, (c, m, _) in enumerate(CASES)])
def test_backward_parity(cid, m, kw):
    import torch
    say("backward", cid, m, kw)
    wl = make_workload(cid, m, 0, **kw)
    dy = draw_dy(wl, 1)
    ffn = make_ffn(wl)
    x = to_dev(wl, wl.x)
    sa = sel_args(wl)
    pack = ffn.new_pack(m)
    ffn.forward(x, pack=pack, **sa)
    f, d = wl.f, wl.d
    dw = {k: torch.zeros((f, d), dtype=torch.float32, device="cuda") for k in ("gate", "up", "down")}
    kw2 = {k: v for k, v in sa.items() if k in ("bias", "bias_scalar", "tau")}
    dx = ffn.backward(x, to_dev(wl, dy), pack, dw_gate=dw["gate"], dw_up=dw["up"], dw_down_nm=dw["down"], **kw2)
    torch.cuda.synchronize()
    if cid == "c5":
        assert int(pack.n_dense[0]) > 0                   # routed tokens take part
    if m >= 2048:
        # full size: sampled tokens (routed ones among them) and neurons, each
        # output evaluated on its own by the oracle
        rng = np.random.default_rng(5)
        routed = pack.dense_list[:int(pack.n_dense[0])].cpu().numpy()
        tokens = np.unique(np.concatenate([rng.choice(m, 56, replace=False), routed[:8]]))
        neurons = np.sort(rng.choice(f, 192, replace=False))
        ref = O.backward_sampled(wl, dy, tokens, neurons)
        check_y(y_to_f64(wl, dx[:m])[tokens], ref["dx"], tol=TOL)
        nt = torch.from_numpy(neurons).cuda()
        check_rows(dw["up"][nt].cpu().numpy().astype(np.float64), ref["dw_up"], "dW_up")
        check_rows(dw["gate"][nt].cpu().numpy().astype(np.float64), ref["dw_gate"], "dW_gate")
        check_rows(dw["down"][nt].cpu().numpy().astype(np.float64), ref["dw_down_nm"], "dW_down")
    else:
        ref = O.backward(wl, dy)
        check_y(y_to_f64(wl, dx[:m]), ref["dx"], tol=TOL)
        check_rows(dw["up"].cpu().numpy().astype(np.float64), ref["dw_up"], "dW_up")
        check_rows(dw["gate"].cpu().numpy().astype(np.float64), ref["dw_gate"], "dW_gate")
        check_rows(dw["down"].cpu().numpy().astype(np.float64), ref["dw_down"].T, "dW_down")
    # accumulation: a second call adds the same values (exactly doubles them)
    first = {k: v.clone() for k, v in dw.items()}
    ffn.backward(x, to_dev(wl, dy), pack, dw_gate=dw["gate"], dw_up=dw["up"], dw_down_nm=dw["down"], **kw2)
    torch.cuda.synchronize()
    for k in dw:
        assert torch.equal(dw[k], 2 * first[k]), k


def test_backward_unsupported_configs():
    from activation_sparse_gated_amd import FFNError
    say("backward unsupported")
    for cid, kw in (("c3", dict(d=256, f=1024, rank=32)), ("c4", dict(d=256, f=1024))):
        wl = make_workload(cid, 2, 0, **kw)
        ffn = make_ffn(wl)
        x = to_dev(wl, wl.x)
        pack = ffn.new_pack(2)
        ffn.forward(x, pack=pack, **sel_args(wl))
        with pytest.raises(FFNError):
            ffn.backward(x, to_dev(wl, draw_dy(wl, 0)), pack, workspace=x, **{k: v for k, v in sel_args(wl).items()
                                                                          if k in ("bias", "bias_scalar", "tau")})
