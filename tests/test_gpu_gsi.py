"""GPU parity of the gated subspace (GSI) linear map against the CPU oracle.

"Gated Subspace Inference for Transformer Acceleration", sections 2.1-2.2:
g = V_k^T x, r = x - V_k g, rho = ||r|| / ||x||; rho < eps gives y = M g with
the cached image M = W V_k, otherwise y = W x.

Checked per call: the image (bf16, within one rounding of the exact product
plus the fp32 accumulation bound), rho (fp32 evaluation, within RHO_TOL), the
slow-token list and count (exact for tokens outside the band
|rho - eps| <= RHO_TOL, where either decision is accepted and y is compared
with the oracle's output on the path the GPU took), and y per token within
the workload's relative L2 bound.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

from oracle import gsi_oracle as G
from synth import bf16_bits, round_bf16
from synth.gsi import GSI_CONFIGS, make_gsi, make_gsi_config
from tests.gpu_util import Y_REL_L2, check_y

pytestmark = pytest.mark.gpu

# |rho_gpu - rho| bound: fp32 sums over d and k give an absolute error near
# 1e-5 * ||x|| in ||r|| for these shapes (g to ~k * 2^-24 relative, each
# (V_k g)_j to ~k * 2^-24 of sum |V||g|); 2e-4 leaves a factor of 20.
RHO_TOL = 2e-4


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def dev_bf16(a):
    import torch
    bits = bf16_bits(np.ascontiguousarray(a)).view(np.int16)
    return torch.from_numpy(bits).view(torch.bfloat16).cuda()


def make_gsi_dev(wl, max_m=None):
    from activation_sparse_gated_amd import GsiLinear
    w, vk = dev_bf16(wl.w), dev_bf16(wl.vk)
    return GsiLinear(w, vk, max_m=max(wl.m, 1) if max_m is None else max_m)


def img_ref(wl):
    return round_bf16(G.image(wl.w, wl.vk))


def check_image(lin, wl, rows=None):
    import torch
    torch.cuda.synchronize()
    got = lin.image().float().cpu().numpy().astype(np.float64)
    rows = np.arange(wl.d_out) if rows is None else rows
    e, g = G.image(wl.w[rows], wl.vk), got[rows]
    a = np.abs(wl.w[rows]) @ np.abs(wl.vk)
    # one bf16 rounding (2^-8 relative) of a value within gamma_d of the exact sum
    gam = wl.d * 2.0 ** -24 / (1 - wl.d * 2.0 ** -24)
    bound = 2.0 ** -8 * (np.abs(e) + gam * a) + gam * a
    assert np.all(np.abs(g - e) <= bound), float(np.max(np.abs(g - e) - bound))
    assert np.mean(g == round_bf16(e)) > 0.99


def run_and_check(lin, wl, eps=None, m=None):
    import torch
    eps = wl.eps if eps is None else eps
    m = wl.m if m is None else m
    x = dev_bf16(wl.x[:m]) if m > 0 else dev_bf16(np.zeros((1, wl.d)))
    y, rho, sl, ns = lin.forward(x, eps, m)
    torch.cuda.synchronize()
    if m == 0:
        assert int(ns[0]) == 0
        return None
    img = img_ref(wl)
    y_ref, rho_ref, slow_ref = G.forward(wl.w, img, wl.vk, wl.x[:m], eps)
    rho_g = rho[:m].cpu().numpy().astype(np.float64)
    assert np.all(np.abs(rho_g - rho_ref) <= RHO_TOL), float(np.max(np.abs(rho_g - rho_ref)))
    n = int(ns[0])
    got_slow = sl[:n].cpu().numpy().tolist()
    assert got_slow == sorted(set(got_slow))
    band = np.abs(rho_ref - eps) <= RHO_TOL
    for t in range(m):
        if not band[t]:
            assert (t in got_slow) == (t in set(slow_ref.tolist())), t
    # y against the oracle's output on the path the GPU took for each token
    dense = G.dense(wl.w, wl.x[:m])
    fast = G.project(wl.vk, wl.x[:m])[0] @ img.T
    ref = np.where(np.isin(np.arange(m), got_slow)[:, None], dense, fast)
    yg = y[:m].float().cpu().numpy().astype(np.float64)
    check_y(yg, ref)
    for t in range(m):
        if not np.any(wl.x[t]):
            assert np.all(yg[t] == 0.0)
    return y_ref, got_slow


SMALL = [
    dict(d=64, d_out=40, k=16, m=5, eps=0.3, slow_frac=0.4, seed=0),
    dict(d=200, d_out=77, k=24, m=9, eps=0.2, slow_frac=0.5, seed=1),       # ragged d, k/8 not a power of two
    dict(d=8, d_out=3, k=8, m=2, eps=0.2, slow_frac=0.0, seed=2),           # k = d
    dict(d=1024, d_out=600, k=512, m=16, eps=0.1, slow_frac=0.3, seed=3),   # 64 lanes per k-row
    dict(d=512, d_out=1000, k=64, m=37, eps=0.15, slow_frac=0.25, seed=4),  # three groups of tokens
    dict(d=2048, d_out=513, k=128, m=3, eps=0.1, slow_frac=0.5, seed=5, zero_tokens=(1,)),
    dict(d=4096, d_out=257, k=256, m=8, eps=0.05, slow_frac=0.0, seed=6),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"d{c['d']}-o{c['d_out']}-k{c['k']}-m{c['m']}" for c in SMALL])
def test_gsi_parity_small(case):
    say("gsi small", case)
    kw = dict(case)
    d, d_out, k, m = kw.pop("d"), kw.pop("d_out"), kw.pop("k"), kw.pop("m")
    wl = make_gsi(d, d_out, k, m, **kw)
    lin = make_gsi_dev(wl)
    check_image(lin, wl)
    run_and_check(lin, wl)
    # two more calls on the same handle: fewer tokens, then eps = 0 (all slow)
    run_and_check(lin, wl, m=max(1, m // 2))
    run_and_check(lin, wl, eps=0.0)


def test_gsi_exact_tie_goes_slow():
    """rho == eps exactly (rho = 1/2 in both precisions) takes W x."""
    import torch
    say("gsi tie")
    d, k, d_out = 16, 8, 24
    vk = np.zeros((d, k))
    vk[:k, :k] = np.eye(k)
    x = np.zeros((2, d))
    x[:, :3] = 1.0
    x[:, 8] = 1.0                   # ||r||^2 = 1, ||x||^2 = 4
    wl = make_gsi(d, d_out, k, 2, eps=0.5, basis=vk, seed=7)
    wl.x = x
    lin = make_gsi_dev(wl)
    xd = dev_bf16(x)
    for eps, want in ((0.5, [0, 1]), (float(np.nextafter(np.float32(0.5), np.float32(1))), [])):
        y, rho, sl, ns = lin.forward(xd, eps)
        torch.cuda.synchronize()
        assert rho.cpu().numpy().tolist() == [0.5, 0.5]
        assert sl[:int(ns[0])].cpu().numpy().tolist() == want
        run_and_check(lin, wl, eps=eps)


def test_gsi_full_basis_identity_is_dense():
    """k = d with V_k = I: every token fast, image = W, y = W x."""
    say("gsi identity basis")
    d = 256
    wl = make_gsi(d, 96, d, 6, eps=1e-3, basis=np.eye(d), seed=8)
    lin = make_gsi_dev(wl)
    import torch
    torch.cuda.synchronize()
    img = lin.image().float().cpu().numpy().astype(np.float64)
    assert np.array_equal(img, wl.w)                       # W V with V = I is W, exactly
    _, slow = run_and_check(lin, wl)
    assert slow == []


def test_gsi_zero_tokens_and_errors():
    import torch
    say("gsi zero tokens / errors")
    wl = make_gsi(128, 64, 16, 4, eps=0.2, slow_frac=0.5, seed=9, zero_tokens=(0, 2))
    lin = make_gsi_dev(wl, max_m=4)
    run_and_check(lin, wl)
    run_and_check(lin, wl, m=0)
    x = dev_bf16(wl.x)
    y = lin.new_output(4)
    assert lin.forward_raw(x, 0.2, y, m=5) == -1                 # above max_m
    assert lin.forward_raw(x, float("nan"), y) == -1
    assert lin.forward_raw(x, 0.2, y[:, 1:], m=4) == -1          # misaligned y
    # outputs are optional
    assert lin.forward_raw(x, 0.2, y) == 0
    torch.cuda.synchronize()
    run_and_check(lin, wl)


@pytest.mark.parametrize("m,n_slow", [(1, None), (16, None), (16, 4), (21, 3)])
def test_gsi_full_size(m, n_slow):
    """The LoPA FFN's up projection: d = 4096 -> 14336, k = 256, eps = 0.10."""
    say("gsi full size", m, n_slow)
    wl = make_gsi_config("gsi", m=m, seed=0, n_slow=n_slow)
    lin = make_gsi_dev(wl)
    rows = np.random.default_rng(0).choice(wl.d_out, 512, replace=False)
    check_image(lin, wl, rows=rows)
    run_and_check(lin, wl)


@pytest.mark.parametrize("m", [1, 5, 16])
def test_gsi_dense_forward_full_size(m):
    """The comparison baseline y = W x at the workload's shape."""
    import torch
    say("gsi dense", m)
    wl = make_gsi_config("gsi", m=m, seed=1)
    lin = make_gsi_dev(wl)
    y = lin.dense_forward(dev_bf16(wl.x))
    torch.cuda.synchronize()
    check_y(y[:m].float().cpu().numpy().astype(np.float64), G.dense(wl.w, wl.x))
