"""CPU oracle for the activation-sparse gated FFN forward pass.

TEST INFRASTRUCTURE ONLY. Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this module; the library never does.

A plain, slow evaluation in fp64 of what the sparse path computes, written
from the method's definitions (sources below), one step at a time with no
blocking or fusion. It shares no code with the HIP library. Inputs are the
generator's rounded values (fp32- or bf16-representable), taken as fp64.

Sources (page title, then section):

* LoPA page -- "Meta FAIR and Inria's LoPA Gating Hits 3.31x Real GPU
  Speedup for LLM Inference", section "How LoPA Gating Restructures FFN
  Computation": the gated FFN order (gate projection, activation, elementwise
  product with the value projection, down projection); unstructured,
  per-token sparsity; the low-rank gate with rank ratio 1/8.
* Sparser/Faster/Lighter page -- news.neo-ai.one article 2802 on the
  Sakana AI + NVIDIA paper "Sparser, Faster, Lighter Transformer Language
  Models": section "稀疏不等於提速" (ReLU as the source of unstructured
  sparsity; the gated-FFN formula itself is lost in the page text), section
  "TwELL 減掉轉換開銷" (tile-wise ELLPACK emitted by the gate epilogue; one
  pass computing up and down without storing h), section "Hybrid
  應對非均勻稀疏" (high-activity rows routed to a dense backup).
* WINA page -- "大语言模型推理加速新突破：解读WINA框架的核心原理与实践价值",
  section 3.1 (score = |hidden value| times the 2-norm of the weight column
  it multiplies) and section 3.2 (Lemma 3.1: optimal for column-orthogonal
  weights).
* LoPA page, section "Model Casting and Quality at 90% Sparsity": the gating
  carries over to mixture-of-experts layers whose experts are FFN blocks.
* Sparser/Faster/Lighter page, section "Hybrid 應對非均勻稀疏": in training
  the same hybrid (compact format for most tokens, dense backup for busy
  ones) cuts dense work and stored activations; the backward pass here is
  the gradient of the forward pass with its selection held fixed.

Readings where the pages are silent (each is listed with its reason in the
design notes): y = W_down (a(z) * (W_up x)) with z = W_gate x + b and no
up/down biases; "ReLU with threshold" passes z through (a = z when
z > max(tau, 0)); the low-rank intermediate V x is kept unrounded; a cut is
strict (z == cut is inactive); top-k orders by (score desc, index asc);
a token is routed dense when any tile holds more than E active entries; in a
mixture-of-experts layer each expert is one such FFN and a token's output is
the routing-weighted sum of its chosen experts' outputs.

Parity status: every function below is pinned by CPU tests (brute-force
dense evaluation, closed forms, invariants, the hand-computed WINA example
and a Lemma-3.1 enumeration). The y values themselves have no printed
example on the pages; beyond those pins their tolerance is the one the
workload statement fixes.
"""
from __future__ import annotations

import numpy as np

RELU, SILU = "relu", "silu"
SEL_BIAS, SEL_THRESH, SEL_TOPK = "bias", "thresh", "topk"
IDX_PAD = 0xFFFF


# ---------------------------------------------------------------------------
# rounding of reported pack values
# ---------------------------------------------------------------------------

def bf16_rne_bits(v) -> np.ndarray:
    """bf16 bit pattern nearest to each fp64 value (ties to even).

    Works on the fp64 encoding directly: keep the top 8 significant bits
    (1 implicit + 7 stored), i.e. drop the low 45 of 52 fraction bits with
    round-to-nearest-even; a carry into the exponent is the correct result.
    Then rebias the 11-bit exponent to bf16's 8-bit one.
    """
    v = np.asarray(v, dtype=np.float64)
    bits = np.ascontiguousarray(v).view(np.uint64).copy()
    low_mask = np.uint64((1 << 45) - 1)
    half = np.uint64(1 << 44)
    lsb = (bits >> np.uint64(45)) & np.uint64(1)
    bits = (bits + (half - np.uint64(1)) + lsb) & ~low_mask
    sign = (bits >> np.uint64(63)) & np.uint64(1)
    exp = ((bits >> np.uint64(52)) & np.uint64(0x7FF)).astype(np.int64)
    frac7 = (bits >> np.uint64(45)) & np.uint64(0x7F)
    e8 = exp - 1023 + 127
    zero = (exp == 0) | (e8 <= 0)
    out = (sign << np.uint64(15)) | (np.clip(e8, 0, 255).astype(np.uint64) << np.uint64(7)) | frac7
    out = np.where(zero, sign << np.uint64(15), out)
    return out.astype(np.uint16)


def bf16_bits_to_f64(b) -> np.ndarray:
    """fp64 value of bf16 bit patterns."""
    b = np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# steps of the forward pass
# ---------------------------------------------------------------------------

def gate_preactivation(x, w_gate=None, u=None, v=None) -> np.ndarray:
    """g[t, i] = <W_gate[i, :], x_t>, or for the low-rank gate
    g = U (V x_t) with the rank-r intermediate kept in fp64 (not rounded).

    [LoPA page, "How LoPA Gating Restructures FFN Computation": a gate of
    reduced rank (ratio 1/8) in place of the full gate projection.]
    """
    x = np.asarray(x, dtype=np.float64)
    if w_gate is not None:
        return x @ np.asarray(w_gate, dtype=np.float64).T
    t = x @ np.asarray(v, dtype=np.float64).T        # [m, r], fp64, unrounded
    return t @ np.asarray(u, dtype=np.float64).T


def activation(z, act: str) -> np.ndarray:
    """sigma(z): ReLU, or SiLU z / (1 + exp(-z))."""
    z = np.asarray(z, dtype=np.float64)
    if act == RELU:
        return np.maximum(z, 0.0)
    if act == SILU:
        return z / (1.0 + np.exp(-z))
    raise ValueError(act)


def threshold_mask(z, cut) -> np.ndarray:
    """Active set of a bias / threshold gate: z > cut, strictly (z == cut
    is inactive, as ReLU(0) = 0).

    [Sparser/Faster/Lighter page, "稀疏不等於提速": ReLU zeros give the
    unstructured, token-dependent sparsity.] The cut is 0 in bias mode and
    max(tau_t, 0) in threshold mode (a ReLU output at or below 0 is zero).
    """
    z = np.asarray(z, dtype=np.float64)
    cut = np.asarray(cut, dtype=np.float64)
    return z > cut.reshape(-1, 1) if cut.ndim == 1 else z > cut


def up_projection(x, w_up) -> np.ndarray:
    """u[t, i] = <W_up[i, :], x_t> for every neuron (dense reference)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w_up, dtype=np.float64).T


def wina_column_norms(w_down) -> np.ndarray:
    """c_i = || W_down[:, i] ||_2, the norm of the weight column neuron i feeds.

    [WINA page, section 3.1: the weight part of the score.]
    """
    w = np.asarray(w_down, dtype=np.float64)
    return np.sqrt(np.sum(w * w, axis=0))


def wina_scores(h, col_norms) -> np.ndarray:
    """s_i = |h_i| * c_i. [WINA page, section 3.1.]"""
    return np.abs(np.asarray(h, dtype=np.float64)) * np.asarray(col_norms, dtype=np.float64)


def input_column_norms(w) -> np.ndarray:
    """c_j = || W[:, j] ||_2 for input channel j of a linear layer W
    [out x in]: the weight column that input element j multiplies.

    [WINA page, section 3.1, applied to a layer's input: the weight part of
    the score of input element j.] For the gate projection W is W_gate, or V
    for the low-rank gate U (V x).
    """
    w = np.asarray(w, dtype=np.float64)
    return np.sqrt(np.sum(w * w, axis=0))


def input_scores(x, col_norms) -> np.ndarray:
    """s_j = |x_j| * c_j for every input channel j. [WINA page, section
    3.1; with equal c_j this is the hidden-state magnitude rule of TEAL and
    CATS that section 二 describes.]"""
    return np.abs(np.asarray(x, dtype=np.float64)) * np.asarray(col_norms, dtype=np.float64)


def gate_preactivation_input_sparse(x, kept, w_gate=None, u=None, v=None) -> np.ndarray:
    """Gate pre-activation from the kept input channels only:
    g_t = W_gate[:, S_t] x_t[S_t], or for the low-rank gate
    g_t = U (V[:, S_t] x_t[S_t]) with the rank-r intermediate in fp64.
    kept[t] lists S_t. [WINA page, section 3.1: the input elements outside
    the kept set are treated as zero in the layer they feed.]
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_gate if w_gate is not None else v, dtype=np.float64)
    first = np.stack([w[:, np.asarray(kept[t], dtype=np.int64)] @ x[t, np.asarray(kept[t], dtype=np.int64)]
                      for t in range(x.shape[0])]) if x.shape[0] else np.zeros((0, w.shape[0]))
    if w_gate is not None:
        return first
    return first @ np.asarray(u, dtype=np.float64).T


def topk_lower_index(s_row, k: int) -> np.ndarray:
    """Indices of the k largest scores of one token, ties to the lower
    index, returned in ascending index order."""
    s_row = np.asarray(s_row, dtype=np.float64)
    order = sorted(range(s_row.size), key=lambda i: (-s_row[i], i))
    return np.array(sorted(order[:k]), dtype=np.int64)


def twell_pack(mask, values, T: int, E: int, f32_values: bool):
    """Tile-wise ELLPACK of per-token active values.

    Columns are cut into tiles of T; per (token t, tile j):
    cnt[t, j] = number of active columns in the tile, idx[t, j, :] = the
    first min(cnt, E) active local offsets in ascending order (padding
    0xFFFF), val[t, j, :] = their values (bf16 bits, or fp32 for fp32
    inputs; padding 0).

    [Sparser/Faster/Lighter page, "TwELL 減掉轉換開銷": no global row
    alignment; 1-D tiles of columns matched to the compute tiles.]
    """
    mask = np.asarray(mask, dtype=bool)
    values = np.asarray(values, dtype=np.float64)
    m, f = mask.shape
    nt = f // T
    cnt = np.zeros((m, nt), dtype=np.int32)
    idx = np.full((m, nt, E), IDX_PAD, dtype=np.uint16)
    val = np.zeros((m, nt, E), dtype=np.float32 if f32_values else np.uint16)
    for t in range(m):
        for j in range(nt):
            cols = np.nonzero(mask[t, j * T:(j + 1) * T])[0]
            cnt[t, j] = cols.size
            keep = cols[:E]
            idx[t, j, :keep.size] = keep
            vals = values[t, j * T + keep]
            if f32_values:
                val[t, j, :keep.size] = vals.astype(np.float32)
            else:
                val[t, j, :keep.size] = bf16_rne_bits(vals)
    return cnt, idx, val


def route_tokens(cnt, E: int):
    """route_t = 1 when any tile of token t holds more than E active
    entries; dense_list = the routed token ids in ascending order.

    [Sparser/Faster/Lighter page, "Hybrid 應對非均勻稀疏": rows with many
    non-zeros go to a dense backup path, the rest stay in the compact
    format.]
    """
    cnt = np.asarray(cnt)
    route = (cnt > E).any(axis=1).astype(np.uint8) if cnt.size else np.zeros(cnt.shape[0], np.uint8)
    dense_list = np.nonzero(route)[0].astype(np.int32)
    return route, dense_list, int(dense_list.size)


def down_projection_sparse(h_active, cols, w_down) -> np.ndarray:
    """y = sum over active neurons i of h_i * W_down[:, i] (fp64)."""
    w = np.asarray(w_down, dtype=np.float64)
    if len(cols) == 0:
        return np.zeros(w.shape[0])
    return w[:, cols] @ np.asarray(h_active, dtype=np.float64)


# ---------------------------------------------------------------------------
# the whole forward pass
# ---------------------------------------------------------------------------

def forward(wl, k: int | None = None, E: int | None = None, T: int | None = None,
            bias=None, tau=None) -> dict:
    """Sparse forward pass of one workload instance.

    Returns a dict with g (pre-bias gate), z, mask, act_values (a, or h in
    top-k mode), cnt, idx, val, route, dense_list, n_dense, y (fp64
    [m, d]) and, in top-k mode, scores and topk index lists.
    [Sparser/Faster/Lighter page, "TwELL 減掉轉換開銷": only the active
    neurons' up rows and down columns enter the result.]
    """
    T = wl.T if T is None else T
    E = wl.E if E is None else E
    k = wl.k if k is None else k
    m, f = wl.m, wl.f
    x = np.asarray(wl.x, dtype=np.float64)
    b = wl.bias_per_token() if bias is None else np.asarray(bias, dtype=np.float64)
    out = {}
    k_in = getattr(wl, "in_keep", 0) or 0
    if k_in:
        # input-side selection of the gate projection: the k_in input channels
        # with the largest |x_j| * ||W[:, j]||_2 (ties to the lower index)
        c_in = input_column_norms(wl.w_gate if wl.w_gate is not None else wl.v)
        s_in = input_scores(x, c_in)
        kept = [topk_lower_index(s_in[t], k_in) for t in range(m)]
        g = gate_preactivation_input_sparse(x, kept, wl.w_gate, wl.u, wl.v)
        out.update(in_norms=c_in, in_scores=s_in, in_kept=kept)
    else:
        g = gate_preactivation(x, wl.w_gate, wl.u, wl.v)
    z = g + b.reshape(-1, 1)
    out.update(g=g, z=z)

    if wl.sel == SEL_TOPK:
        a = activation(z, wl.act)
        u = up_projection(x, wl.w_up)                 # top-k needs u for every neuron
        h = a * u
        c = wina_column_norms(wl.w_down)
        s = wina_scores(h, c)
        mask = np.zeros((m, f), dtype=bool)
        sets = []
        for t in range(m):
            sel = topk_lower_index(s[t], k)
            sets.append(sel)
            mask[t, sel] = True
        packed_vals = h
        y = np.stack([down_projection_sparse(h[t, mask[t]], np.nonzero(mask[t])[0], wl.w_down)
                      for t in range(m)]) if m else np.zeros((0, wl.d))
        out.update(scores=s, col_norms=c, topk=sets, h=h, u=u)
    else:
        if wl.act != RELU:
            raise ValueError("bias / threshold selection is defined for a ReLU gate")
        if wl.sel == SEL_BIAS:
            cut = np.zeros(m)
        else:
            t_in = wl.tau if tau is None else np.asarray(tau, dtype=np.float64)
            cut = np.maximum(t_in, 0.0)
        mask = threshold_mask(z, cut)
        packed_vals = np.where(mask, z, 0.0)          # a = ReLU(z) = z on active entries
        y = np.zeros((m, wl.d))
        for t in range(m):
            cols = np.nonzero(mask[t])[0]
            u_act = np.asarray(wl.w_up, dtype=np.float64)[cols] @ x[t]   # only active up rows
            y[t] = down_projection_sparse(z[t, cols] * u_act, cols, wl.w_down)
    cnt, idx, val = twell_pack(mask, packed_vals, T, E, wl.dtype == "f32")
    route, dense_list, n_dense = route_tokens(cnt, E)
    out.update(mask=mask, act_values=packed_vals, cnt=cnt, idx=idx, val=val, route=route,
               dense_list=dense_list, n_dense=n_dense, y=y)
    return out


def dense_forward(wl, bias=None, tau=None) -> np.ndarray:
    """The same function evaluated densely over every neuron.

    Bias / threshold gates keep their elementwise mask; a top-k gate keeps
    every neuron (the unsparsified FFN it approximates). The gate reads every
    input channel (no input-side selection).
    """
    x = np.asarray(wl.x, dtype=np.float64)
    b = wl.bias_per_token() if bias is None else np.asarray(bias, dtype=np.float64)
    z = gate_preactivation(x, wl.w_gate, wl.u, wl.v) + b.reshape(-1, 1)
    a = activation(z, wl.act)
    if wl.sel == SEL_THRESH:
        t_in = wl.tau if tau is None else np.asarray(tau, dtype=np.float64)
        a = np.where(threshold_mask(z, np.maximum(t_in, 0.0)), a, 0.0)
    h = a * up_projection(x, wl.w_up)
    return h @ np.asarray(wl.w_down, dtype=np.float64).T


# ---------------------------------------------------------------------------
# backward pass (training)
# ---------------------------------------------------------------------------

def backward(wl, dy, fwd: dict | None = None) -> dict:
    """Gradients of L = sum_t <dy_t, y_t> through the sparse forward pass with
    its selection held fixed (full-rank ReLU gate, bias or threshold rule).

    With a = z on the active entries (0 elsewhere), u = W_up x, h = a * u and
    y = W_down h: dh = W_down^T dy; du = dh * a; dz = dh * u on the active
    entries; dW_down = dy h^T; dW_up = du x^T; dW_gate = dz x^T;
    dx = W_up^T du + W_gate^T dz. Only the active neurons' rows and columns
    are non-zero. [Sparser/Faster/Lighter page, "Hybrid 應對非均勻稀疏":
    training with the hybrid format; the chain rule through the gated FFN
    order of the LoPA page, "How LoPA Gating Restructures FFN Computation".]
    Returns dx [m, d], dw_gate [f, d], dw_up [f, d], dw_down [d, f]
    (output-major, as W_down) and the per-token du, dz, h [m, f].
    """
    if wl.sel == SEL_TOPK or wl.w_gate is None:
        raise ValueError("the backward pass is defined here for a full-rank ReLU gate with a bias or threshold")
    fwd = forward(wl) if fwd is None else fwd
    x = np.asarray(wl.x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    w_down = np.asarray(wl.w_down, dtype=np.float64)
    mask = fwd["mask"]
    a = np.where(mask, fwd["z"], 0.0)
    u = up_projection(x, wl.w_up)
    h = a * u
    dh = dy @ w_down                                 # row t: W_down^T dy_t
    du = dh * a
    dz = np.where(mask, dh * u, 0.0)
    return {
        "dx": du @ np.asarray(wl.w_up, dtype=np.float64) + dz @ np.asarray(wl.w_gate, dtype=np.float64),
        "dw_gate": dz.T @ x,
        "dw_up": du.T @ x,
        "dw_down": dy.T @ h,
        "du": du, "dz": dz, "h": h, "mask": mask,
    }


def backward_sampled(wl, dy, tokens, neurons) -> dict:
    """The outputs of `backward` for a sample, by the same definitions: dx of
    the given tokens, and the gradient rows of the given neurons. A token's
    dx needs its own z, mask, u and dh over every neuron; a neuron's gradient
    rows need that neuron's z, mask, u and dh over every token. The mask is
    the bias / threshold rule on z (a routed token keeps the same mask: its
    dense gate evaluates the same selection). [Sources as for `backward`.]
    Returns dx [len(tokens), d], and for the neurons dw_gate, dw_up and
    dw_down_nm (row i = dW_down[:, i]), each [len(neurons), d]."""
    if wl.sel == SEL_TOPK or wl.w_gate is None or wl.act != RELU:
        raise ValueError("the backward pass is defined here for a full-rank ReLU gate with a bias or threshold")
    x = np.asarray(wl.x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    w_gate = np.asarray(wl.w_gate, dtype=np.float64)
    w_up = np.asarray(wl.w_up, dtype=np.float64)
    w_down = np.asarray(wl.w_down, dtype=np.float64)
    b = wl.bias_per_token()
    cut = np.zeros(wl.m) if wl.sel == SEL_BIAS else np.maximum(np.asarray(wl.tau, dtype=np.float64), 0.0)
    tk = np.asarray(tokens, dtype=np.int64)
    nr = np.asarray(neurons, dtype=np.int64)
    # the sampled tokens over every neuron
    z_t = gate_preactivation(x[tk], w_gate) + b[tk].reshape(-1, 1)
    m_t = threshold_mask(z_t, cut[tk])
    a_t = np.where(m_t, z_t, 0.0)
    u_t = up_projection(x[tk], w_up)
    dh_t = dy[tk] @ w_down
    du_t = dh_t * a_t
    dz_t = np.where(m_t, dh_t * u_t, 0.0)
    # the sampled neurons over every token
    z_n = gate_preactivation(x, w_gate[nr]) + b.reshape(-1, 1)
    m_n = threshold_mask(z_n, cut)
    a_n = np.where(m_n, z_n, 0.0)
    u_n = up_projection(x, w_up[nr])
    dh_n = dy @ w_down[:, nr]
    du_n = dh_n * a_n
    dz_n = np.where(m_n, dh_n * u_n, 0.0)
    return {
        "dx": du_t @ w_up + dz_t @ w_gate,
        "dw_gate": dz_n.T @ x,
        "dw_up": du_n.T @ x,
        "dw_down_nm": (a_n * u_n).T @ dy,
    }


# ---------------------------------------------------------------------------
# mixture of experts
# ---------------------------------------------------------------------------

def moe_combine(expert_y, rows, slots, weights, m: int, d: int) -> np.ndarray:
    """y_t = sum over token t's routing slots s of weights[t, s] times the
    output of the expert of slot s on x_t. expert_y[e] holds expert e's
    outputs for its tokens rows[e] (routing slots slots[e]). [LoPA page,
    "Model Casting and Quality at 90% Sparsity": experts are FFN blocks; the
    weighted sum is the usual combination of a routed layer.]"""
    y = np.zeros((m, d))
    w = np.asarray(weights, dtype=np.float64)
    for ye, r_e, s_e in zip(expert_y, rows, slots):
        for i, (t, s) in enumerate(zip(r_e, s_e)):
            y[int(t)] += w[int(t), int(s)] * np.asarray(ye[i], dtype=np.float64)
    return y


def moe_forward(mw) -> dict:
    """Each expert's sparse forward pass on the tokens routed to it, then the
    weighted combination. Returns the per-expert results and y [m, d]."""
    per = [forward(wl) if wl.m else None for wl in mw.experts]
    ys = [p["y"] if p is not None else np.zeros((0, mw.d)) for p in per]
    return {"experts": per, "y": moe_combine(ys, mw.rows, mw.slots, mw.weights, mw.m, mw.d)}
