"""Muon, NorMuon and AdamW optimizer steps -- oracle (test infrastructure only).

[nanochat] "5만원으로 나만의 ChatGPT 훈련하는 방법", section "2. Muon optimizer
(nanochat/optim.py)": a matrix parameter's update is orthogonalized by five
quintic Newton-Schulz steps ("Polar Express"), and after that NorMuon
normalizes the update per neuron so its scale does not collapse.

What the orthogonalization computes.  A step with coefficients (a, b, c)
replaces X by the odd quintic of X, aX + bX(X^T X) + cX(X^T X)^2.  For
X = U S V^T (thin SVD) that matrix is U p(S) V^T with p(s) = a s + b s^3 +
c s^5 applied to every singular value: the singular vectors never change,
only the singular values move through the composition of the steps'
polynomials.  That is the definition used here in fp64 (`polar_express`):
one SVD of the normalised start, the composed polynomial on its singular
values.  The page prints two of its five coefficient tuples, so the tuples
are an input.

READINGS (the page shows the idea, not every detail):
  * start: X = G / (||G||_F + eps), eps = 1e-7 (the polynomials are built for
    singular values in [0, 1]; Muon's normalisation);
  * bf16 mode (the rounding points of a bf16 implementation, which cannot
    take an SVD): the quintic is formed through the Gram matrix of the
    smaller side, A = X^T X, as X p_(A) with p_(A) = aI + bA + cA^2; X, A and
    p_(A) are stored as bf16 between the products, the products themselves
    exact;
  * orientation: for a matrix with fewer rows than columns the Gram matrix
    is taken on the row side (X X^T); the result is the same in exact
    arithmetic, and the fp64 form does not depend on it.
"""
from __future__ import annotations

import numpy as np

from .gpt import round_bf16

NS_EPS = 1e-7


def _rnd(x, bf16: bool):
    return round_bf16(np.asarray(x, np.float32)).astype(np.float64) if bf16 else x


def quintic(s, coeffs):
    """The composition of the steps' odd polynomials s -> a s + b s^3 + c s^5,
    applied elementwise."""
    s = np.asarray(s, np.float64)
    for a, b, c in coeffs:
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def polar_express(G, coeffs, eps: float = NS_EPS, bf16: bool = False) -> np.ndarray:
    """The orthogonalized update of G [m, n]: exact (fp64, through the SVD of
    the normalised start), or with bf16 storage of X, A and p_(A) when bf16
    is set."""
    G = np.asarray(G, np.float64)
    X0 = G / (np.linalg.norm(G) + eps)
    if not bf16:
        U, S, Vt = np.linalg.svd(X0, full_matrices=False)
        return (U * quintic(S, coeffs)) @ Vt
    if G.shape[0] < G.shape[1]:
        return polar_express(G.T, coeffs, eps, bf16).T
    X = _rnd(X0, True)
    eye = np.eye(X.shape[1])
    for a, b, c in coeffs:
        A = _rnd(X.T @ X, True)
        P = _rnd(a * eye + b * A + c * (A @ A), True)
        X = _rnd(X @ P, True)
    return X


def ns_flops(m: int, n: int, steps: int) -> float:
    """Multiply-add flops of the Gram-matrix form: per step X^T X (2 m n^2),
    A A (2 n^3) and X p_(A) (2 m n^2), with n the smaller side."""
    m, n = max(m, n), min(m, n)
    return steps * (4.0 * m * n * n + 2.0 * n ** 3)


# --------------------------------------------------------------------------
# NorMuon: per-neuron normalisation of the orthogonalized update
# --------------------------------------------------------------------------
# The page's snippet takes the mean square of the update over `red_dim`
# (one value per neuron), the root of the sum of those means (v_norm), and
# multiplies the update by step_size * v_norm / v_norm_new, the last clamped
# below at 1e-10; it leaves red_dim, step_size and v_norm_new undefined.
# READINGS (NorMuon as published: an Adam-style second moment per neuron,
# then the overall size restored):
#   * neuron = output row of the [out, in] weight: red_dim is the input
#     (column) axis, v_mean[r] = mean_c X[r, c]^2;
#   * step_size[r] = 1 / sqrt(max(v[r], 1e-10)), v the per-row second moment
#     kept across steps, v <- beta2 v + (1 - beta2) v_mean (zero before the
#     first step, no bias correction);
#   * v_norm_new = the same quantity as v_norm for the update scaled by
#     step_size: sqrt(sum_r v_mean[r] step_size[r]^2);
#   * the scale multiplies the update in fp32 (the update is consumed by the
#     parameter step directly, with no rounding in between).
# With these, ||X * final_scale||_F = ||X||_F whenever v_norm_new > 1e-10:
# NorMuon only redistributes the update's size across neurons.
NORMUON_FLOOR = 1e-10


def normuon(X, v, beta2: float):
    """(X scaled per row, the new per-row second moment v), fp64."""
    X = np.asarray(X, np.float64)
    v_mean = np.mean(X * X, axis=1)
    v = beta2 * np.asarray(v, np.float64) + (1.0 - beta2) * v_mean
    step_size = 1.0 / np.sqrt(np.maximum(v, NORMUON_FLOOR))
    v_norm = np.sqrt(np.sum(v_mean))
    v_norm_new = np.sqrt(np.sum(v_mean * step_size ** 2))
    final_scale = step_size * (v_norm / max(v_norm_new, NORMUON_FLOOR))
    return X * final_scale[:, None], v


# --------------------------------------------------------------------------
# the elementwise parts of the optimizer step
# --------------------------------------------------------------------------
# READINGS: the page names Muon (momentum, orthogonalized update) for the
# block matrices and AdamW for embeddings, lm_head and value embeddings, and
# prints neither the momentum form nor the AdamW constants, so the published
# definitions are used with every constant an argument: Muon's momentum
# buffer M <- beta M + (1 - beta) G with the Nesterov look-ahead
# (1 - beta) G + beta M as the update fed to the orthogonalization; the
# parameter step W <- W (1 - lr wd) - lr X (decoupled decay, lr carrying any
# shape factor; X after NorMuon when it is on); AdamW as Loshchilov & Hutter
# with bias correction.

def muon_momentum(grad, mom, beta: float, nesterov: bool = True):
    """(new momentum, the update to orthogonalize), fp64."""
    grad = np.asarray(grad, np.float64)
    m = beta * np.asarray(mom, np.float64) + (1.0 - beta) * grad
    return m, ((1.0 - beta) * grad + beta * m) if nesterov else m


def muon_update(w, x, lr: float, wd: float):
    """W (1 - lr wd) - lr X."""
    return np.asarray(w, np.float64) * (1.0 - lr * wd) - lr * np.asarray(x, np.float64)


def adamw(w, grad, m, v, step: int, lr: float, beta1: float, beta2: float, eps: float,
          wd: float):
    """One AdamW step (step counts from 1): returns (w, m, v)."""
    g = np.asarray(grad, np.float64)
    m = beta1 * np.asarray(m, np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, np.float64) + (1.0 - beta2) * g * g
    mhat = m / (1.0 - beta1 ** step)
    vhat = v / (1.0 - beta2 ** step)
    w = np.asarray(w, np.float64) * (1.0 - lr * wd) - lr * mhat / (np.sqrt(vhat) + eps)
    return w, m, v
