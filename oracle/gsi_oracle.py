"""CPU oracle for the gated-subspace fast path of a linear map (GSI).

TEST INFRASTRUCTURE ONLY. Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this module; the library never does.

A plain evaluation in fp64 of what the GSI entry points compute, written from
the method's definitions, one step at a time. It shares no code with the HIP
library. Inputs are the generator's bf16-rounded values, taken as fp64.

Source (page title, then section): "Gated Subspace Inference for Transformer
Acceleration",
* section 2.1 (core decomposition): for a linear map y = W x with W of shape
  d_out x d and an orthonormal rank-k basis V_k (d x k), the input splits
  exactly into x = V_k (V_k^T x) + r, so y = (W V_k)(V_k^T x) + W r = M g + W r
  with the cached low-rank image M = W V_k and the projection g = V_k^T x;
* section 2.2 (gated residual pass-through): per token, the residual ratio
  rho = ||r|| / ||x||; below the threshold eps the output is taken as M g
  (the fast path reads only the image), otherwise (rho >= eps) the full
  product W x is computed; Theorem 4 bounds the fast path's error by
  ||W||_2 * eps * ||x||.

Readings where the page is silent (each is listed in the design notes):
* the image is cached at the weights' precision: the caller of `forward`
  passes the image it holds (the library keeps bf16); `image` returns it
  unrounded;
* g is kept unrounded between the projection and the image product;
* a token with x = 0 has rho = 0 (0/0 read as "no residual"): it takes the
  fast path, and both paths give y = 0 there;
* V_k is used as given: r is x - V_k V_k^T x even when rounding has left the
  basis only nearly orthonormal (the decomposition stays exact by that
  definition);
* tokens are independent: the slow-path list is the slow tokens in
  increasing order.

Parity status: every function is pinned by CPU tests (a hand-computed toy
with printed expected values, brute-force loops, the eps = 0 and k = d
reductions to the dense product, Pythagoras for an orthonormal basis and the
Theorem-4 bound).
"""
from __future__ import annotations

import numpy as np


def image(w: np.ndarray, vk: np.ndarray) -> np.ndarray:
    """Low-rank weight image M = W V_k (d_out x k), GSI page section 2.1."""
    w = np.asarray(w, dtype=np.float64)
    vk = np.asarray(vk, dtype=np.float64)
    return w @ vk


def project(vk: np.ndarray, x: np.ndarray):
    """Projection and residual of each token (rows of x), section 2.1.

    Returns g = V_k^T x per token (m x k), r = x - V_k g (m x d) and the
    residual ratio rho = ||r|| / ||x|| of section 2.2 (0 for a zero token).
    """
    vk = np.asarray(vk, dtype=np.float64)
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    g = x @ vk                      # row t: V_k^T x_t
    r = x - g @ vk.T                # row t: x_t - V_k g_t
    nr = np.sqrt(np.sum(r * r, axis=1))
    nx = np.sqrt(np.sum(x * x, axis=1))
    rho = np.zeros(x.shape[0])
    nz = nx > 0
    rho[nz] = nr[nz] / nx[nz]
    return g, r, rho


def slow_tokens(rho: np.ndarray, eps: float) -> np.ndarray:
    """Tokens that take the full product: rho >= eps (section 2.2), ascending."""
    return np.nonzero(~(np.asarray(rho, dtype=np.float64) < float(eps)))[0].astype(np.int64)


def dense(w: np.ndarray, x: np.ndarray) -> np.ndarray:
    """The plain linear map y = W x per token (the slow path), m x d_out."""
    w = np.asarray(w, dtype=np.float64)
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    return x @ w.T


def forward(w: np.ndarray, img: np.ndarray, vk: np.ndarray, x: np.ndarray, eps: float):
    """Gated GSI output of every token, section 2.2.

    Fast tokens (rho < eps): y = M g with the image `img` as cached;
    slow tokens: y = W x. Returns (y [m x d_out], rho [m], slow list).
    """
    g, _, rho = project(vk, x)
    slow = slow_tokens(rho, eps)
    img = np.asarray(img, dtype=np.float64)
    y = g @ img.T                   # fast path for every token ...
    if slow.size:
        y[slow] = dense(w, np.atleast_2d(np.asarray(x, dtype=np.float64))[slow])   # ... replaced where slow
    return y, rho, slow
