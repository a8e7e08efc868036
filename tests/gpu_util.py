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
                     wdown_out_major=wdown_out_major, in_keep=getattr(wl, "in_keep", 0))


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


# ---------------------------------------------------------------------------
# forward error bounds of the kernels' fp32 arithmetic
#
# A dot product of exact products p_j (bf16 x bf16 is exact in fp32) summed in
# fp32 with every term passing through at most D roundings is off by at most
# gamma_D * sum_j |p_j|, gamma_D = D u / (1 - D u), u = 2**-24 (for fp32
# operands one more rounding per product: D + 1). Every gate / up summation of
# the library has depth D <= K / 32 + 32 for a contraction of length K: the
# VALU GEMVs chain 8 fused multiply-adds per 512-element piece over at most 8
# pieces and add a 6-level wave butterfly (K / 64 + 6); the matrix-core tiles
# accumulate K / 32 chunk products in sequence, at most 5 levels inside one
# MFMA, and at most 16 wave, slab or split-K partials. The fp32 (tiny
# workload) kernels are bounded by D = K + 1 instead.
# ---------------------------------------------------------------------------
U32 = 2.0 ** -24


def gamma(D: int) -> float:
    return D * U32 / (1.0 - D * U32)


def _depth(wl, K: int) -> int:
    return K + 1 if wl.dtype == "f32" else K // 32 + 32


def gate_error_bound(wl) -> np.ndarray:
    """[m, f] bound on |g_gpu - g| for the gate pre-activation.

    Full gate: gamma_D * sum_j |W_gate[i, j] x_j|. Low rank: t = V x carries
    e_t = gamma_D1 * |V| |x|; the second stage multiplies U by t split into
    bf16 hi + lo (|t - hi - lo| <= 2**-17 |t|) or by fp32 t in the VALU, so
    the bound is |U| e_t + |U| (|t| + e_t) (2**-17 + gamma_D2 (1 + 2**-8)),
    with D2 = 2 r / 32 + 32 (two MFMA passes per chunk).
    """
    xs = np.asarray(wl.x, dtype=np.float64)
    d1 = _depth(wl, wl.d)
    if getattr(wl, "in_keep", 0):
        # the input-side gate reads only the kept channels (the oracle's
        # selection) and sums their products in channel groups, in any
        # order: depth d + 1
        from oracle import ffn_oracle as O
        c_in = O.input_column_norms(wl.w_gate if wl.w_gate is not None else wl.v)
        s_in = O.input_scores(xs, c_in)
        keep = np.zeros_like(xs)
        for t_ in range(xs.shape[0]):
            keep[t_, O.topk_lower_index(s_in[t_], wl.in_keep)] = 1.0
        xs = xs * keep
        d1 = wl.d + 1
    x = np.abs(xs)
    if wl.w_gate is not None:
        return gamma(d1) * (x @ np.abs(wl.w_gate).T)
    t = xs @ np.asarray(wl.v, dtype=np.float64).T
    e_t = gamma(d1) * (x @ np.abs(wl.v).T)
    au = np.abs(np.asarray(wl.u, dtype=np.float64))
    d2 = wl.rank + 1 if wl.dtype == "f32" else 2 * wl.rank // 32 + 32
    return 1.01 * (e_t @ au.T + ((np.abs(t) + e_t) @ au.T) * (2.0 ** -17 + gamma(d2) * (1 + 2.0 ** -8)))


def score_error_bound(wl, ref) -> np.ndarray:
    """[m, f] bound on |s_gpu - s| for the WINA score s = |SiLU(g + b) u| c.

    e_g, e_u: the dot-product bounds of the gate and up rows; SiLU is
    1.1-Lipschitz and is evaluated within 8 u relative; h = a u adds one
    rounding; c = ||W_down[:, i]||_2 sums d squares (depth d / 64 + 6, all
    terms positive) and takes a correctly rounded square root; s adds one
    more rounding. First-order terms, times 1.01 for the products of error
    terms.
    """
    x = np.abs(np.asarray(wl.x, dtype=np.float64))
    D = _depth(wl, wl.d)
    e_g = gamma(D) * (x @ np.abs(wl.w_gate).T) + U32 * np.abs(ref["z"])
    e_u = gamma(D) * (x @ np.abs(wl.w_up).T)
    z = ref["z"]
    a = z / (1.0 + np.exp(-z))
    uu = ref["u"]
    e_a = 1.1 * e_g + 8 * U32 * (np.abs(a) + 1.1 * e_g)
    e_h = e_a * (np.abs(uu) + e_u) + np.abs(a) * e_u + U32 * (np.abs(a) + e_a) * (np.abs(uu) + e_u)
    c = ref["col_norms"]
    e_c = (gamma(wl.d // 64 + 6) / 2 + 2 * U32) * c
    h = np.abs(ref["h"])
    return 1.01 * ((c + e_c) * e_h + h * e_c + U32 * (h + e_h) * (c + e_c))


def check_scores(wl, s_gpu, ref, m=None):
    """WINA scores: every GPU score within the forward error bound of its
    fp32 evaluation (score_error_bound) of the fp64 score."""
    m = wl.m if m is None else m
    bound = score_error_bound(wl, ref)
    err = np.abs(s_gpu[:m].astype(np.float64) - ref["scores"][:m])
    bad = err > bound[:m]
    assert not bad.any(), (f"{int(bad.sum())} scores outside the error bound; worst "
                           f"err/bound {float(np.max(err / np.maximum(bound[:m], 1e-300))):.3g}")
    return float(np.max(err / np.maximum(bound[:m], 1e-300)))


def check_gate_band(wl, g_gpu: np.ndarray, ref, m=None):
    """The GPU gate stays within its forward error bound (gate_error_bound) and
    within a quarter of the certified guard band. Returns the largest error
    as a fraction of rms(g) over the tokens."""
    m = wl.m if m is None else m
    err = np.abs(g_gpu[:m].astype(np.float64) - ref["g"][:m])
    bound = gate_error_bound(wl)[:m]
    bad = err > bound
    assert not bad.any(), f"{int(bad.sum())} gate values outside the forward error bound"
    worst = 0.0
    for t in range(m):
        rms = float(np.sqrt(np.mean(ref["g"][t] ** 2)))
        if rms > 0:
            worst = max(worst, float(err[t].max()) / rms)
        if wl.delta[t] > 0:
            assert err[t].max() <= wl.delta[t] / 4, f"token {t}: gate error {err[t].max():.3e} > delta/4"
    return worst
