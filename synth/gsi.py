"""Seeded synthetic inputs for the gated subspace (GSI) linear map.

The pages measure the method on model activations that lie close to a
low-dimensional subspace; no such activations exist here, so each token is
built as a subspace part plus an orthogonal residual of a chosen relative
size:

* W [d_out, d] ~ N(0, 1/d), rounded to bf16;
* the basis V_k [d, k]: the orthonormal Q factor of an N(0, 1) matrix (fp64),
  rounded to bf16 (so only nearly orthonormal, as a cached bf16 basis is);
* token t: p = Q c with c ~ N(0, I_k); n = e - Q (Q^T e) with e ~ N(0, I_d),
  scaled so that ||n|| / ||p + n|| is the token's target ratio; x = p + n,
  scaled to unit rms and rounded to bf16.

Target ratios are drawn away from the threshold: fast tokens in
[0.2, 0.8] * eps, slow tokens in [1.5, 6] * eps (capped below 1). The bf16
rounding of x and V_k moves a token's ratio by about 1e-3 of ||x||, far
less than those margins; nothing here evaluates the method itself.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .workloads import round_bf16

# streams
_S_W, _S_BASIS, _S_SLOW, _S_RATIO, _S_C, _S_E = range(1, 7)
_GSI_ID = 40


def _rng(*path) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(p) for p in path]))


@dataclass
class GsiWorkload:
    """One seeded instance (fp64 values on the bf16 grid)."""
    name: str
    d: int
    d_out: int
    k: int
    m: int
    eps: float
    w: np.ndarray          # [d_out, d]
    vk: np.ndarray         # [d, k]
    x: np.ndarray          # [m, d]
    target: np.ndarray     # [m] target residual ratio of each token
    slow_target: np.ndarray  # [m] bool: drawn as a slow token


# Workloads: the LoPA FFN's up projection (d = 4096 -> 14336) with the
# rank and threshold of the page's GPT-J working point (k = 256,
# eps = 0.10, 99.8% of tokens on the fast path).
GSI_CONFIGS = {
    "gsi": dict(name="gsi-linear-bf16-4096x14336-k256", d=4096, d_out=14336, k=256, ms=(1, 16),
                eps=0.10, slow_frac=0.002),
}


def make_gsi(d: int, d_out: int, k: int, m: int, *, eps: float = 0.10, slow_frac: float = 0.25,
             seed: int = 0, n_slow: int | None = None, zero_tokens=(), name: str = "gsi",
             basis: np.ndarray | None = None, w_scale: float = 1.0) -> GsiWorkload:
    """Draw W, V_k and m tokens. `n_slow` fixes the number of slow tokens
    (placed at random positions); otherwise each token is slow with
    probability `slow_frac`. `zero_tokens` are set to x = 0."""
    if not (1 <= k <= d):
        raise ValueError("need 1 <= k <= d")
    w = round_bf16(_rng(_GSI_ID, seed, _S_W, d, d_out).standard_normal((d_out, d)) * (w_scale / np.sqrt(d)))
    if basis is None:
        a = _rng(_GSI_ID, seed, _S_BASIS, d, k).standard_normal((d, k))
        q, _ = np.linalg.qr(a)
    else:
        q = np.asarray(basis, dtype=np.float64)
    vk = round_bf16(q)
    rs = _rng(_GSI_ID, seed, _S_SLOW, m)
    if n_slow is None:
        slow = rs.random(m) < slow_frac
    else:
        slow = np.zeros(m, dtype=bool)
        slow[rs.permutation(m)[:n_slow]] = True
    rr = _rng(_GSI_ID, seed, _S_RATIO, m).random(m)
    target = np.where(slow, np.minimum(eps * (1.5 + 4.5 * rr), 0.95), eps * (0.2 + 0.6 * rr))
    x = np.zeros((m, d))
    for t in range(m):
        if t in zero_tokens:
            target[t] = 0.0
            slow[t] = False
            continue
        c = _rng(_GSI_ID, seed, _S_C, t).standard_normal(q.shape[1])
        p = q @ c
        e = _rng(_GSI_ID, seed, _S_E, t).standard_normal(d)
        n = e - q @ (q.T @ e)
        nn, pn = np.linalg.norm(n), np.linalg.norm(p)
        rho = target[t]
        if nn > 0 and rho > 0:
            n *= rho * pn / np.sqrt(1.0 - rho * rho) / nn
        else:
            n[:] = 0.0
        v = p + n
        v *= np.sqrt(d) / max(np.linalg.norm(v), 1e-300)
        x[t] = round_bf16(v)
    return GsiWorkload(name=name, d=d, d_out=d_out, k=k, m=m, eps=eps, w=w, vk=vk, x=x,
                       target=target, slow_target=slow)


def make_gsi_config(cid: str, m: int | None = None, seed: int = 0, **kw) -> GsiWorkload:
    cfg = GSI_CONFIGS[cid]
    mm = cfg["ms"][0] if m is None else m
    kw.setdefault("slow_frac", cfg["slow_frac"])
    return make_gsi(cfg["d"], cfg["d_out"], cfg["k"], mm, eps=cfg["eps"], seed=seed, name=cfg["name"], **kw)
