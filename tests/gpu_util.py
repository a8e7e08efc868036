"""Helpers for GPU parity tests: device copies of generator arrays and the
comparisons against the CPU oracle (tolerances in one place)."""
from __future__ import annotations

import numpy as np

Y_REL_L2 = 5e-3          # per-token relative L2 bound on y (workload statement)


def to_dev(wl, a):
    import torch
    if a is None:
        return None
    if wl.dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    bits = wl.storage(a).view(np.int16)
    return torch.from_numpy(bits).view(torch.bfloat16).cuda()


def f32_dev(a):
    import torch
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def make_ffn(wl, max_m=None, wdown_out_major=True, E=None, T=None):
    from activation_sparse_gated_amd import SparseFFN
    w_down = wl.w_down if wdown_out_major else np.ascontiguousarray(wl.w_down.T)
    return SparseFFN(d_model=wl.d, d_ff=wl.f, rank=wl.rank, dtype=wl.dtype, act=wl.act, sel=wl.sel,
                     tile_w=wl.T if T is None else T, ell_w=wl.E if E is None else E,
                     max_m=max(wl.m, 1) if max_m is None else max_m,
                     w_gate=to_dev(wl, wl.w_gate), u=to_dev(wl, wl.u), v=to_dev(wl, wl.v),
                     w_up=to_dev(wl, wl.w_up), w_down=to_dev(wl, w_down),
                     wdown_out_major=wdown_out_major)


def sel_args(wl, bias=None, tau=None):
    """Keyword arguments of gate_pack / forward for a workload."""
    kw = {}
    if bias is not None:
        kw["bias"] = f32_dev(bias)
    elif wl.bias is not None:
        kw["bias"] = f32_dev(wl.bias)
    else:
        kw["bias_scalar"] = 0.0 if wl.bias_scalar is None else wl.bias_scalar
    if wl.sel == "thresh":
        kw["tau"] = f32_dev(wl.tau if tau is None else tau)
    if wl.sel == "topk":
        kw["k"] = wl.k
    return kw


def host(t):
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def y_to_f64(wl, y):
    import torch
    if wl.dtype == "f32":
        return y.detach().cpu().numpy().astype(np.float64)
    return y.detach().float().cpu().numpy().astype(np.float64)


def check_y(y_gpu: np.ndarray, y_ref: np.ndarray, tol: float = Y_REL_L2, rows=None):
    rows = range(y_ref.shape[0]) if rows is None else rows
    worst = 0.0
    for t in rows:
        nr = np.linalg.norm(y_ref[t])
        if nr == 0.0:
            assert np.all(y_gpu[t] == 0.0), f"token {t}: reference row is zero, GPU row is not"
            continue
        rel = np.linalg.norm(y_gpu[t] - y_ref[t]) / nr
        worst = max(worst, rel)
        assert rel <= tol, f"token {t}: rel L2 {rel:.3e} > {tol}"
    return worst


def check_pack(wl, pack, ref, m=None, E=None):
    """cnt / idx / route / dense_list bit-exact. Values: both sides round the
    same pre-activation (z = g + b, or h) to the storage type, from fp32 on the
    GPU and fp64 in the oracle, so they may differ by one unit in the last
    place of the rounded value plus the gate's own error, bounded by the
    certified delta/4 (z = g + b can cancel near the cut)."""
    m = wl.m if m is None else m
    E = wl.E if E is None else E
    cnt = host(pack.cnt)[:m]
    assert np.array_equal(cnt, ref["cnt"]), "cnt differs"
    route = host(pack.route)[:m]
    assert np.array_equal(route, ref["route"]), "route differs"
    nd = int(host(pack.n_dense)[0])
    assert nd == ref["n_dense"], f"n_dense {nd} != {ref['n_dense']}"
    assert np.array_equal(host(pack.dense_list)[:nd], ref["dense_list"]), "dense_list differs"
    if E == 0:
        return
    idx = host(pack.idx)[:m].view(np.uint16)
    assert np.array_equal(idx, ref["idx"]), "idx differs"
    val = host(pack.val)[:m]
    if wl.dtype == "f32":
        gv = val.astype(np.float64)
        rv = ref["val"].astype(np.float64)
        ulp = np.spacing(np.abs(ref["val"]).astype(np.float32)).astype(np.float64)
    else:
        from oracle.ffn_oracle import bf16_bits_to_f64
        gv = bf16_bits_to_f64(val)
        rv = bf16_bits_to_f64(ref["val"])
        _, ex = np.frexp(rv)                    # |rv| in [2**(ex-1), 2**ex): bf16 ulp 2**(ex-8)
        ulp = np.where(rv == 0.0, 0.0, np.ldexp(1.0, ex - 8))
    band = np.zeros(m) if wl.sel == "topk" else np.asarray(wl.delta[:m]) / 4.0
    tol = ulp + band.reshape(-1, 1, 1)
    bad = np.abs(gv - rv) > tol
    assert not bad.any(), f"{int(bad.sum())} pack values outside 1 ulp + delta/4"


def check_scores(wl, s_gpu, ref, m=None):
    """WINA scores: every GPU score stays on its side of the top-k cut, with
    at least half of its distance to the cut (and half of the certified
    half-gap) to spare."""
    m = wl.m if m is None else m
    k = wl.k
    for t in range(m):
        sr = ref["scores"][t]
        if not 0 < k < wl.f:
            continue
        srt = np.sort(sr)[::-1]
        cut = 0.5 * (srt[k - 1] + srt[k])
        half_gap = 0.5 * (srt[k - 1] - srt[k])
        err = np.abs(s_gpu[t].astype(np.float64) - sr)
        lim = np.maximum(0.5 * half_gap, 0.5 * np.abs(sr - cut))
        assert np.all(err <= lim), f"token {t}: score error crosses the top-k cut margin"


def check_gate_band(wl, g_gpu: np.ndarray, ref, m=None):
    """The GPU gate stays within a quarter of the certified guard band."""
    m = wl.m if m is None else m
    err = np.abs(g_gpu[:m].astype(np.float64) - ref["g"][:m])
    for t in range(m):
        if wl.delta[t] > 0:
            assert err[t].max() <= wl.delta[t] / 4, f"token {t}: gate error {err[t].max():.3e} > delta/4"
    return float(err.max())
